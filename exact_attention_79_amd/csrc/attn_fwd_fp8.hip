// attn_fwd_fp8.hip -- fp8 (OCP e4m3) forward kernel for gfx950.
//
// Method: the same tiled online-softmax forward as attn_fwd.hip (FLASH-ATTN
// page, FlashAttention-2 section), with both products on the fp8 matrix
// cores as in the "Low-precision with FP8" part of the page's
// FlashAttention-3 summary: Q, K, V arrive as e4m3 codes with one descale
// per tensor; the score scale becomes s * dq * dk, and dv multiplies the
// output once in the epilogue.
//
// Probabilities are requantised to e4m3 for the P V product with a scale per
// (query row, 64-key block): the row's largest probability in the block sets
// a power-of-two scale 2^e that brings it into [128, 256), so every entry
// keeps the full 3-bit mantissa of e4m3's normal range.  One e4m3 term
// leaves a relative weight error of up to 2^-4, which on inputs with outlier
// channels exceeds the accuracy asked of this path; P is therefore carried
// as two e4m3 terms, x = P 2^-e = hi + 2^-4 lo with lo = e4m3(16 (x - hi)),
// giving a relative error of about 2^-8 for one extra fp8 product.  The
// scales are not applied on the VALU: v_mfma_scale_f32_32x32x64_f8f6f4 takes
// a per-lane E8M0 block scale for its B operand, and lane l's block is
// exactly the 32 probabilities of one query that it holds, so the matrix
// core multiplies by 2^e (hi) and 2^(e-4) (lo) itself.
//
// Layout (mirrors the bf16 kernel): each wave owns 32 queries and computes
// S^T = K Q^T (keys on M); the C layout gives one query per lane; the fp32
// probabilities, rounded to e4m3 and packed four per register, are the B
// operand of O^T += V^T P^T.  For that operand a lane holds 32 keys of its
// query (16 from each of the two 32-key halves of the block).  V is stored
// in LDS with its rows permuted inside each 64-key block so that the 32 keys
// of each wave half are 32 consecutive rows, which ds_read_b64_tr_b8 reads
// as 8-key columns straight into the A-operand layout.
#include "attn_device.hpp"
#include "attn_kernels.hpp"

namespace attn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short v2i16 __attribute__((ext_vector_type(2)));

// fp8 tiles: rows of D bytes in 16-byte chunks, chunk c of row r at c ^ swz8(r).
// d = 128 (8 chunks, 2 rows per 256-byte bank span): the 16 rows of a row
// read land on 16 different slots, and the 8 rows x 2 chunks of a
// transposing read land on 16 different slots.  d = 64 likewise with 4 rows
// per span.
template <int D>
__device__ __forceinline__ int swz8(int r);
template <>
__device__ __forceinline__ int swz8<128>(int r) {
  return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}
template <>
__device__ __forceinline__ int swz8<64>(int r) {
  return (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
}
template <int D>
__device__ __forceinline__ int off8(int r, int ch) {
  return r * D + ((ch ^ swz8<D>(r)) << 4);
}

// Row of V key `key` inside its LDS tile: within each 64-key block, keys
// 8a + 4b + c (b in {0,1}) go to row 32b + 4a + c, so wave half b finds its
// keys {8a + 4b + c} in 32 consecutive rows.  vkey is the inverse map.
__device__ __forceinline__ int vkey(int row) {
  return (row & ~63) | (((row >> 2) & 7) << 3) | (((row >> 5) & 1) << 2) | (row & 3);
}

// Direct global -> LDS load of rows row0 .. row0+ROWS-1 of a [rows][D] byte
// head (head_bytes long) by NW waves: wave w's instruction i fills LDS chunks
// (i*NW + w)*64 + lane, i.e. chunk ch of LDS row r, which holds global chunk
// ch ^ swz8(r) of source row r (K) or of source row vkey(r) (V, PERMUTE).
// The buffer resource starts at row row0 (scalar arithmetic), so each lane's
// offset is the same for every tile.  Rows past the head's end read as zero.
template <int D, int ROWS, int NW, bool PERMUTE>
__device__ __forceinline__ void tile_load_lds8(const uint8_t* head, uint32_t head_bytes,
                                               int row0, uint8_t* t, int w, int lane) {
  constexpr int CH = D / 16;
  constexpr int ROUNDS = ROWS * CH / (64 * NW);
  static_assert((ROWS * CH) % (64 * NW) == 0 && ROWS % 64 == 0, "tile split");
  const uint32_t rows = head_bytes / D, r0 = (uint32_t)row0;
  const auto rs = make_rsrc(head + (size_t)r0 * D, r0 < rows ? head_bytes - r0 * D : 0u);
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int base = (i * NW + w) * 64;
    const int pc = base + lane, r = pc / CH, ch = (pc % CH) ^ swz8<D>(r);
    const int g = PERMUTE ? vkey(r) : r;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(t + base * 16), 16,
                                             (int)((uint32_t)(g * D + ch * 16)), 0, 0, 0);
  }
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c, int scale_b) {
  // Formats: A and B e4m3 (0); A block scale 2^0 (127); B block scale per lane.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0,
                                                        scale_b);
}

struct FwdFp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  void* o;
  float* lse;
  int H, Hkv;       // query heads per batch element; key/value heads
  int N;
  int n_qtiles;
  float scale;      // softmax scale s
  // Descales: one per tensor (q_descale, k_descale, v_descale), or, when
  // the arrays are given, one per block: qs[b*H+h][query block of BR rows],
  // ks and vs [b*Hkv+h][key block of BC rows].
  float q_descale, k_descale, v_descale;
  const float* qs;
  const float* ks;
  const float* vs;
  int causal, window, out_f32;
};

template <int D, int NW, bool BLOCKS>
__global__ __launch_bounds__(NW * 64, 2) void fwd_fp8_kernel(FwdFp8Params p) {
  constexpr int BC = 64;  // keys per tile = one 64-deep fp8 MFMA step
  constexpr int BR = 32 * NW;
  constexpr int KS = D / 64;  // K-steps of a score tile
  // Three LDS slots each for K and V (tile u in slot u % 3), as separate
  // arrays so that the compiler can tell the slots being filled from the
  // ones being read; tiles are fetched two iterations before first use.
  __shared__ __attribute__((aligned(16))) uint8_t sK0[BC * D];
  __shared__ __attribute__((aligned(16))) uint8_t sK1[BC * D];
  __shared__ __attribute__((aligned(16))) uint8_t sK2[BC * D];
  __shared__ __attribute__((aligned(16))) uint8_t sV0[BC * D];
  __shared__ __attribute__((aligned(16))) uint8_t sV1[BC * D];
  __shared__ __attribute__((aligned(16))) uint8_t sV2[BC * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int h = lane >> 5, n = lane & 31;
  const TileId id =
      tile_order(blockIdx.x, gridDim.x / p.n_qtiles, p.n_qtiles, p.causal, 0);
  const int bh = id.bh;
  const int qt = p.causal ? p.n_qtiles - 1 - id.rank : id.rank;  // longest first
  const int N = p.N;
  const int q0 = qt * BR;
  const int wq0 = q0 + 32 * w;
  const int my_q = wq0 + n;
  const size_t head = (size_t)bh * N * D;
  const size_t kv_off = (size_t)kv_head(bh, p.H, p.Hkv) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D;
  const auto rq = make_rsrc(p.q + head, head_bytes);
  const uint8_t* kh = p.k + kv_off;
  const uint8_t* vh = p.v + kv_off;

  // Q^T as the B operand of S^T = K Q^T: in K-step ks a lane holds the 32
  // bytes d = 64 ks + 32 h .. +31 of its query; K rows are read the same way.
  i32x8 qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)(my_q * D + 64 * ks + 32 * h);
    const u32x4 a = buf_load16(rq, off), b = buf_load16(rq, off + 16);
    qop[ks] = (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                      (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  }

  const int q_last = min(q0 + BR, N) - 1;
  int kv_lo = 0, kv_hi = N;
  if (p.causal) kv_hi = min(kv_hi, q_last + 1);
  if (p.window > 0) {
    kv_lo = max(0, q0 - p.window + 1);
    if (!p.causal) kv_hi = min(kv_hi, q_last + p.window);
  }
  const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = (f32x16){};
  // The running max M is kept in base-2 logit units (s * q.k * log2 e), so
  // that tiles with different key descales compare directly: tile t's raw
  // code products are scaled by s2t(t) = s2q * dk(t).
  float m_run = kMaxInit, l_run = 0.f;
  const int kvh = kv_head(bh, p.H, p.Hkv);
  const int n_kt = (N + BC - 1) / BC;
  const float s2q = p.scale * kLog2e * (BLOCKS ? p.qs[(size_t)bh * p.n_qtiles + qt] : p.q_descale);
  const float s2k = s2q * p.k_descale;  // per-tensor key descale
  auto s2t = [&](int t) {
    return BLOCKS ? s2q * p.ks[(size_t)kvh * n_kt + min(t, n_kt - 1)] : s2k;
  };
  // With block descales, log2 of tile t's value descale, folded into the
  // weights of that tile; a per-tensor value descale is applied once in the
  // epilogue instead (exactly).
  auto vlog = [&](int t) {
    return BLOCKS ? __builtin_amdgcn_logf(p.vs[(size_t)kvh * n_kt + min(t, n_kt - 1)]) : 0.f;
  };

  // K row reads: the A operand of K-step ks for M-tile mt (32 bytes of row
  // 32 mt + n: chunks 4 ks + 2 h and 4 ks + 2 h + 1).
  auto kread = [&](const uint8_t* Ks, int mt, int ks) {
    const int r = 32 * mt + n;
    const u32x4 a = *(const u32x4*)&Ks[off8<D>(r, 4 * ks + 2 * h)];
    const u32x4 b = *(const u32x4*)&Ks[off8<D>(r, 4 * ks + 2 * h + 1)];
    return (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                   (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  };
  // V^T reads: lane j of a 16-lane group reads row (j >> 1) of an 8-row slab,
  // 8 bytes at column 8 (j & 1) of a 16-byte chunk, and receives column
  // (lane & 15) of the slab; four slabs make the A operand of d-tile dt.
  const int trj = lane & 15, trg = lane >> 4;
  const int tr_row = 32 * (trg >> 1) + (trj >> 1);
  const int tr_col = 16 * (trg & 1) + 8 * (trj & 1);
  auto vread = [&](const uint8_t* Vs, int dt) {
    i32x8 va;
#pragma unroll
    for (int t8 = 0; t8 < 4; ++t8) {
      const int row = tr_row + 8 * t8, col = 32 * dt + tr_col;
      const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (LDS_AS i32x2*)&Vs[off8<D>(row, col >> 4) + (col & 15)]);
      va[2 * t8] = x[0];
      va[2 * t8 + 1] = x[1];
    }
    return va;
  };
  auto scores = [&](const uint8_t* Ks, f32x16* sacc) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[mt] = mfma_fp8(kread(Ks, mt, ks), qop[ks], sacc[mt], 127);
    }
  };

  int hi_key = N - 1, lo_key = 0;
  if (p.causal) hi_key = min(hi_key, my_q);
  if (p.window > 0) {
    lo_key = my_q - p.window + 1;
    if (!p.causal) hi_key = min(hi_key, my_q + p.window - 1);
  }
  // Masks tile t element by element when it straddles a boundary of this
  // wave (a uniform test); returns whether it did.  Register r of M-tile mt
  // holds key t*BC + 32mt + 8(r/4) + 4h + r%4.
  auto mask_tile = [&](int t, f32x16* sacc) -> bool {
    const int kv0 = t * BC;
    bool need = kv0 + BC > N;
    if (p.causal) need |= kv0 + BC - 1 > wq0;
    if (p.window > 0) {
      need |= wq0 + 31 - kv0 >= p.window;
      if (!p.causal) need |= kv0 + BC - 1 - wq0 >= p.window;
    }
    if (!need) return false;
    const int lim_hi = hi_key - kv0 - 4 * h, lim_lo = lo_key - kv0 - 4 * h;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * mt + 8 * (r >> 2) + (r & 3);
        sacc[mt][r] = (c > lim_hi || c < lim_lo) ? -__builtin_inff() : sacc[mt][r];
      }
    return true;
  };
  auto tile_max = [&](const f32x16* sacc) {
    float mx = sacc[0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
    return mx;
  };
  // Running max update for a tile whose in-lane raw max is mx and whose
  // scale is st; returns the tile's row max in logit units (both halves).
  // The max only moves when it grows by more than 8 (2^8 in weight).
  auto update_max = [&](float mx, float st) {
    mx = halves_max(mx) * st;
    const float m_new = (mx > m_run + 8.f) ? mx : m_run;
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    }
    return mx;
  };

  tile_load_lds8<D, BC, NW, false>(kh, head_bytes, t_lo * BC, sK0, w, lane);
  tile_load_lds8<D, BC, NW, true>(vh, head_bytes, t_lo * BC, sV0, w, lane);
  tile_load_lds8<D, BC, NW, false>(kh, head_bytes, (t_lo + 1) * BC, sK1, w, lane);
  tile_load_lds8<D, BC, NW, true>(vh, head_bytes, (t_lo + 1) * BC, sV1, w, lane);
  tile_load_lds8<D, BC, NW, false>(kh, head_bytes, (t_lo + 2) * BC, sK2, w, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 scur[2];
  scores(sK0, scur);
  mask_tile(t_lo, scur);
  float tmx = update_max(tile_max(scur), s2t(t_lo));
  // Every wave has read K_0 before the first iteration refills its slot.
  __syncthreads();

  constexpr int kLoadsPerIter = 2 * (BC * D / 16) / (64 * NW);
  constexpr int kWaitOlderLoads = waitcnt_vm(kLoadsPerIter);

  // One iteration for tile t (scores masked in scur, row max tmx, running
  // max already in m_run): reads K_{t+1} from Kr and V_t from Vr, refills
  // Kf (K_t's slot) with K_{t+3} and Vf (V_{t-1}'s slot) with V_{t+2}.
  auto iteration = [&](int t, const uint8_t* Kr, const uint8_t* Vr, uint8_t* Kf,
                       uint8_t* Vf) {
    tile_load_lds8<D, BC, NW, false>(kh, head_bytes, (t + 3) * BC, Kf, w, lane);
    tile_load_lds8<D, BC, NW, true>(vh, head_bytes, (t + 2) * BC, Vf, w, lane);
    // Weights of this tile, times its value descale dv: the row's largest
    // one, 2^y (y = tmx - M + log2 dv), is brought into [128, 256) by 2^-e,
    // e = floor(y) - 7; both factors are folded into the exponent of every
    // weight, and the MFMA's block scale 2^e puts 2^e back.
    const float s2 = s2t(t), lv = vlog(t);
    const float y = fmaxf(BLOCKS ? tmx - m_run + lv : tmx - m_run, -200.f);
    const int e = max(-123, min(127, (int)floorf(y) - 7));
    const float mbe = m_run + (float)e - lv;

    // Bundles 0..NS-1: the next tile's score MFMAs, each with a slice of
    // this tile's weights (exp2 and the e4m3 hi terms); then this tile's
    // P V MFMAs, the hi terms of all D/32 d-tiles first, each with a slice
    // of the 16x residual lo terms, then the lo terms, each with a slice of
    // the next tile's row max.  (Every accumulator still adds hi before lo.
    // Forming the lo terms beside the hi products rather than the score
    // products moves about 40 % of the vector work out of the score bundles;
    // measured 1-4 % faster.)
    constexpr int NS = 2 * KS;
    constexpr int NP = 2 * (D / 32);
    constexpr int WPB = 8 / NS;  // packed words (4 weights) per score bundle
    // Row-max slices of an odd size, so that each is a chain of v_max3 (an
    // even count starts with a two-operand max whose operands the compiler
    // must first quiet); NCH of the lo-term P V bundles take one.
    constexpr int CH = ((32 + (NP - D / 32) - 1) / (NP - D / 32)) | 1;
    constexpr int NCH = (32 + CH - 1) / CH;
    static_assert(WPB >= 1 && 8 % NS == 0, "bundle split");
    static_assert(NCH <= NP - D / 32, "max slices");
    f32x16 snext[2];
    snext[0] = snext[1] = (f32x16){};
    i32x8 ka[NS], va[D / 32], phi, plo;
    float lsum, part[NCH];
    ka[0] = kread(Kr, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    float xs[8][4];  // this tile's weights, kept for their lo terms
    // lo = e4m3(16 (x - hi)) of packed word wd: the scaled convert divides
    // by 2^-4 itself.
    auto lo_terms = [&](int wd) {
      const int hw = phi[wd];
      const float* x = xs[wd];
      const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
      const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
      v2i16 lw = __builtin_bit_cast(v2i16, x[3]);
      lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw, x[0] - h01[0], x[1] - h01[1], 0.0625f,
                                                    false);
      lw = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lw, x[2] - h23[0], x[3] - h23[1], 0.0625f,
                                                    true);
      plo[wd] = __builtin_bit_cast(int, lw);
    };
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + 1 < NS) ka[i + 1] = kread(Kr, (i + 1) / KS, (i + 1) % KS);
      if (i == NS - 1) va[0] = vread(Vr, 0);
      snext[i / KS] = mfma_fp8(ka[i], qop[i % KS], snext[i / KS], 127);
#pragma unroll
      for (int u = 0; u < WPB; ++u) {
        const int wd = WPB * i + u, mt = wd >> 2, r0 = 4 * (wd & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xs[wd][j] = fast_exp2(fmaf(scur[mt][r0 + j], s2, -mbe));
          lsum = (wd == 0 && j == 0) ? xs[wd][j] : lsum + xs[wd][j];  // (no 0 + x)
        }
        // (The first convert of each pair writes the low word and keeps the
        // high one, which the second convert then fills: any old value will
        // do, so an existing register is passed instead of a zeroed one.)
        int hw = __builtin_bit_cast(int, xs[wd][3]);
        hw = __builtin_amdgcn_cvt_pk_fp8_f32(xs[wd][0], xs[wd][1], hw, false);
        hw = __builtin_amdgcn_cvt_pk_fp8_f32(xs[wd][2], xs[wd][3], hw, true);
        phi[wd] = hw;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    constexpr int LPB = 8 / (D / 32);  // lo words per hi bundle
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const bool lo = j >= D / 32;
      const int dt = lo ? j - D / 32 : j;
      if (!lo && dt + 1 < D / 32) va[dt + 1] = vread(Vr, dt + 1);
      oacc[dt] = mfma_fp8(va[dt], lo ? plo : phi, oacc[dt], lo ? e - 4 + 127 : e + 127);
      if (!lo) {
#pragma unroll
        for (int u = 0; u < LPB; ++u) lo_terms(LPB * j + u);
      }
      if (j >= D / 32 && j - D / 32 < NCH) {
        const int c = j - D / 32;
        float mx = snext[(c * CH) >> 4][(c * CH) & 15];
#pragma unroll
        for (int u = 1; u < CH; ++u) {
          const int el = c * CH + u;
          if (el < 32) mx = fmaxf(mx, snext[el >> 4][el & 15]);
        }
        // Pinned here: it is only read after the loop, and the compiler
        // would otherwise sink it there, out of the bundles.
        asm volatile("" ::"v"(mx));
        part[c] = mx;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // l sums the weights themselves: lsum 2^e / dv.
    l_run += BLOCKS ? __builtin_ldexpf(lsum, e) * fast_exp2(-lv) : __builtin_ldexpf(lsum, e);
    if (t + 1 < t_hi) {
      float mx = part[0];
#pragma unroll
      for (int c = 1; c < NCH; ++c) mx = fmaxf(mx, part[c]);
      if (mask_tile(t + 1, snext)) mx = tile_max(snext);
      tmx = update_max(mx, s2t(t + 1));
    }
    // The loads issued one iteration ago (K_{t+2}, V_{t+1}) have landed for
    // this wave; after the barrier they have for every wave, and the slots
    // read in this iteration may be refilled.
    __builtin_amdgcn_s_waitcnt(kWaitOlderLoads);
    __builtin_amdgcn_s_barrier();
    scur[0] = snext[0];
    scur[1] = snext[1];
  };

  for (int t = t_lo; t < t_hi; t += 3) {
    iteration(t, sK1, sV0, sK0, sV2);
    if (t + 1 < t_hi) iteration(t + 1, sK2, sV1, sK1, sV0);
    if (t + 2 < t_hi) iteration(t + 2, sK0, sV2, sK2, sV1);
  }
  __builtin_amdgcn_s_waitcnt(0);

  const float l_tot = halves_sum(l_run);
  if (my_q < N) {
    const float inv = (BLOCKS ? 1.f : p.v_descale) / l_tot;
    const size_t row = head + (size_t)my_q * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        const float x0 = oacc[dt][4 * g + 0] * inv, x1 = oacc[dt][4 * g + 1] * inv;
        const float x2 = oacc[dt][4 * g + 2] * inv, x3 = oacc[dt][4 * g + 3] * inv;
        if (p.out_f32) {
          *(f32x4*)((float*)p.o + row + d0) = (f32x4){x0, x1, x2, x3};
        } else {
          *(bf16x4*)((__bf16*)p.o + row + d0) =
              (bf16x4){(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
        }
      }
    if (h == 0 && p.lse)
      p.lse[(size_t)bh * N + my_q] =
          (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

template <int D>
static hipError_t launch_fp8_d(const FwdArgs& a, hipStream_t stream, const char** name) {
  constexpr int NW = 4;
  FwdFp8Params p;
  p.q = (const uint8_t*)a.q;
  p.k = (const uint8_t*)a.k;
  p.v = (const uint8_t*)a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.H = a.H;
  p.Hkv = a.Hkv;
  p.N = a.N;
  p.n_qtiles = (a.N + 32 * NW - 1) / (32 * NW);
  p.scale = a.scale;
  p.q_descale = a.q_descale;
  p.k_descale = a.k_descale;
  p.v_descale = a.v_descale;
  p.qs = a.q_scales;
  p.ks = a.k_scales;
  p.vs = a.v_scales;
  p.causal = a.causal;
  p.window = a.window;
  p.out_f32 = a.out_f32;
  const unsigned grid = (unsigned)(a.BH * p.n_qtiles);
  if (a.q_scales)
    return go<fwd_fp8_kernel<D, NW, true>>(name, kname("attn::fwd_fp8_kernel", D, NW, true),
                                           dim3(grid), dim3(NW * 64), stream, p);
  return go<fwd_fp8_kernel<D, NW, false>>(name, kname("attn::fwd_fp8_kernel", D, NW, false),
                                          dim3(grid), dim3(NW * 64), stream, p);
}

hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream, const char** name) {
  if (a.d == 128) return launch_fp8_d<128>(a, stream, name);
  return launch_fp8_d<64>(a, stream, name);
}

}  // namespace attn

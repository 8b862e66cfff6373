// attn_fwd.hip -- bf16 and fp8-input forward kernels for gfx950.
//
// Method (FLASH-ATTN page, FlashAttention-2 section): one workgroup owns a
// block of B_r queries and walks the K/V blocks of its head in order, keeping
// per query a running max m, a running sum l and an unnormalised output
// O~ <- diag(e^{m_old - m_new}) O~ + e^{S - m_new} V; O = O~ / l and
// L = m + log(l) are written once at the end.  Blocks wholly hidden by the
// causal mask or the window are never loaded; only the blocks that straddle
// the mask boundary evaluate the mask element by element (the "Parallelism"
// and causal-mask paragraphs of that section).  Parallelism is over batch x
// heads x query blocks, with no communication between workgroups.
//
// gfx950 mapping.
//  * Each wave owns 32 queries and computes S^T = K_j Q_i^T on
//    v_mfma_f32_32x32x16_bf16 (keys on the M side, queries on N), so the C
//    layout gives every lane ONE query: the row max and row sum are in-lane
//    reductions plus one exchange between the two wave halves, and the
//    rescale factor is a per-lane scalar.
//  * The probabilities P^T, converted to bf16 in place, are directly the B
//    operand of O^T += V_j^T P^T (d on the M side).  V_j^T is read from LDS
//    with ds_read_b64_tr_b16 using the key permutation of the C layout
//    (see attn_device.hpp), so nothing moves between lanes.
//  * Q_i^T stays in VGPRs for the whole K/V loop; K_j and V_j stream
//    through a ring of three LDS slots, filled by direct global -> LDS loads
//    issued two to three tiles ahead of use, with one barrier per tile.
//  * Scores stay in raw units; exp2 takes fma(S, s*log2e, -m*s*log2e).  The
//    running max is only moved when a new score exceeds it by more than
//    8 / (s*log2e) (i.e. 2^8 in probability units): every exponent stays
//    <= 2^8, far inside fp32/bf16 range, and the result is the same exact
//    softmax because the numerator and l use the same reference value.
//  * LDS rows are XOR-swizzled in 16-byte chunks (attn_device.hpp) so that
//    the row-wise 128-bit reads of K and the transposing reads of V are free
//    of bank conflicts.
//  * Workgroups are renumbered per XCD (whole heads per XCD, sharing K/V in
//    that XCD's L2) and, with the causal mask, the longest query blocks run
//    first.
// fwd_bf16_kernel serves dropout and grids of fewer than four 256-query
// workgroups; otherwise the forward runs fwd_pp_kernel below, which keeps
// this mapping but separates each wave's matrix and vector work into
// alternating half-steps (ping-pong).  fwd_fp8_pp_kernel is the same kernel
// for e4m3 inputs (the FlashAttention-3 summary's "Low-precision with FP8"
// part), which it widens in LDS.
#include "attn_device.hpp"
#include "attn_kernels.hpp"

namespace attn {

struct FwdKParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  void* o;
  float* lse;
  int H, Hkv;  // query heads per batch element; key/value heads
  int N;
  int n_qtiles;
  float scale;
  int causal, window, out_f32;
  Dropout drop;
  // e4m3 inputs (fwd_pp_kernel with IN > 0; q, k, v then point at codes):
  // descales per tensor, or per block (IN = 2): qs [BH][ceil(N/128)], ks and
  // vs [B*Hkv][ceil(N/64)].
  float q_descale, k_descale, v_descale;
  const float* qs;
  const float* ks;
  const float* vs;
};

// DROP: dropout on P (the keep bytes of attn_device.hpp); l and L stay those
// of the undropped probabilities, and the 1 / keep scale is applied with 1 / l.
template <int D, int NW, int BC, bool DROP>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(FwdKParams p) {
  constexpr int BR = 32 * NW;  // queries per workgroup
  static_assert(BC == 32 || BC == 64, "the pipeline is written for 32- or 64-key tiles");
  // Three LDS slots each for K and V, as separate arrays so that the
  // compiler can tell the tiles being filled from the tiles being read.
  // Tile u (counted from the first visible tile) lives in slot u % 3; tiles
  // are fetched two iterations before they are first read.
  __shared__ __attribute__((aligned(16))) __bf16 sK0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sK1[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sK2[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV1[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV2[BC * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int h = lane >> 5, n = lane & 31;
  // With the causal mask the last query blocks are the longest: run them first.
  const TileId id =
      tile_order(blockIdx.x, gridDim.x / p.n_qtiles, p.n_qtiles, p.causal, causal_group<D>());
  const int bh = id.bh;
  const int qt = p.causal ? p.n_qtiles - 1 - id.rank : id.rank;
  const int N = p.N;
  const int q0 = qt * BR;
  const int wq0 = q0 + 32 * w;             // first query of this wave
  const int my_q = wq0 + n;                // this lane's query
  const size_t head = (size_t)bh * N * D;
  const size_t kv_off = (size_t)kv_head(bh, p.H, p.Hkv) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc(p.q + head, head_bytes);
  const __bf16* kh = p.k + kv_off;
  const __bf16* vh = p.v + kv_off;

  // Q^T as the B operand of S^T = K Q^T: K-step ks covers d = 16ks..16ks+15,
  // lane holds d = 16ks + 8h .. +7 of its query (zero beyond N).
  bf16x8 qop[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qop[ks] = __builtin_bit_cast(
        bf16x8, buf_load16(rq, (uint32_t)(my_q * D + 16 * ks + 8 * h) * 2u));

  // Keys this workgroup can see at all.
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
  float m_run = kMaxInit, l_run = 0.f;
  const float s2 = p.scale * kLog2e;
  const float tau = 8.0f / s2;
  const TrCoord trc(lane);  // transposing-read coordinates of this lane

  // S^T = K_j Q_i^T (raw scores, fp32), keys on M, this wave's queries on N.
  auto scores = [&](const __bf16* Ks, f32x16* sacc) {
#pragma unroll
    for (int mt = 0; mt < BC / 32; ++mt) {
      sacc[mt] = (f32x16){};
      const int r = 32 * mt + n;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        sacc[mt] = mfma32(tile_row8<D>(Ks, r, 2 * ks + h), qop[ks], sacc[mt]);
    }
  };

  // Keys this lane may see: lo_key <= key <= hi_key.
  int hi_key = N - 1, lo_key = 0;
  if (p.causal) hi_key = min(hi_key, my_q);
  if (p.window > 0) {
    lo_key = my_q - p.window + 1;
    if (!p.causal) hi_key = min(hi_key, my_q + p.window - 1);
  }

  // Masks the scores of tile t element by element, but only when the tile
  // straddles a boundary of this wave (a uniform test); returns whether it
  // did.  Register r of M-tile mt holds key t*BC + 32mt + 8(r/4) + 4h + r%4.
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
    for (int mt = 0; mt < BC / 32; ++mt)
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
    for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
    return mx;
  };

  // Moves the running max to cover a new tile whose in-lane max is mx (the
  // max only moves when it grows by more than tau), rescaling O~ and l.
  auto update_max = [&](float mx) {
    mx = halves_max(mx);
    const float m_new = (mx > m_run + tau) ? mx : m_run;
    const float alpha = fast_exp2((m_run - m_new) * s2);
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    }
  };

  // Prologue: K_0..K_2 and V_0, V_1 in flight (u = tile - t_lo), then S
  // and the running max for the first tile.  Tiles past the last visible
  // one may be loaded and scored: rows past N read as zeros and their
  // scores are never used.
  tile_load_lds<D, BC, NW>(kh, head_bytes, t_lo * BC, sK0, w, lane);
  tile_load_lds<D, BC, NW>(vh, head_bytes, t_lo * BC, sV0, w, lane);
  tile_load_lds<D, BC, NW>(kh, head_bytes, (t_lo + 1) * BC, sK1, w, lane);
  tile_load_lds<D, BC, NW>(vh, head_bytes, (t_lo + 1) * BC, sV1, w, lane);
  tile_load_lds<D, BC, NW>(kh, head_bytes, (t_lo + 2) * BC, sK2, w, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 scur[BC / 32];
  scores(sK0, scur);
  mask_tile(t_lo, scur);
  update_max(tile_max(scur));
  // Every wave has read K_0 before the first iteration refills its slot.
  __syncthreads();

  // vmcnt <= the loads issued by one iteration (lgkmcnt and expcnt free).
  constexpr int kLoadsPerIter = 2 * (BC * D / 8) / (64 * NW);
  constexpr int kWaitOlderLoads = (kLoadsPerIter & 0xF) | (0x7 << 4) | (0xF << 8) |
                                  ((kLoadsPerIter >> 4) << 14);

  // One iteration for tile t, whose scores (masked) are in scur and whose
  // running max is already in m_run: it reads K_{t+1} from Kr and V_t from
  // Vr, and refills Kf (K_t's slot) with K_{t+3} and Vf (V_{t-1}'s slot)
  // with V_{t+2}.  It leaves S_{t+1} (masked) in scur and its max in m_run.
  auto iteration = [&](int t, const __bf16* Kr, const __bf16* Vr, __bf16* Kf,
                       __bf16* Vf) {
    tile_load_lds<D, BC, NW>(kh, head_bytes, (t + 3) * BC, Kf, w, lane);
    tile_load_lds<D, BC, NW>(vh, head_bytes, (t + 2) * BC, Vf, w, lane);
    const float mb = m_run * s2;

    // Main block, scheduled by hand in bundles that the compiler may not
    // reorder across (sched_barrier): each bundle issues one MFMA and the
    // LDS read for the MFMA AHEAD bundles later.
    // Bundles 0..NS-1: the next tile's score MFMAs + this tile's exps;
    // bundles NS..NS+NP-1: this tile's P V MFMAs + slices of the next
    // tile's row max (once its score MFMAs have drained).  A tile that
    // needs the mask has its max taken again after masking (rare).
    constexpr int KS = D / 16;                 // K-steps per score tile
    constexpr int NS = (BC / 32) * KS;         // score MFMAs
    constexpr int NP = (BC / 16) * (D / 32);   // P V MFMAs
    constexpr int EPB = BC / 2 / NS;           // exps per lane per bundle
    constexpr int AHEAD = 4;
    constexpr int NV = BC / 2;                 // scores per lane per tile
    constexpr int J0 = 2;                      // first PV bundle with max work
    // Scores per slice, odd so that each slice is a chain of v_max3 (an
    // even count starts with a two-operand max whose operands the compiler
    // must first quiet), and the number of slices that hold any.
    constexpr int CH = ((NV + (NP - J0) - 1) / (NP - J0)) | 1;
    constexpr int NCH = (NV + CH - 1) / CH;
    static_assert(NCH >= 1 && NCH <= NP - J0 && CH * NCH >= NV, "max slices");
    const __bf16* Kn = Kr;
    const __bf16* Vs = Vr;
    auto kread = [&](int i) {
      return tile_row8<D>(Kn, 32 * (i / KS) + n, 2 * (i % KS) + h);
    };
    auto vread = [&](int j) { return tile_a_tr<D>(Vs, trc, j / (D / 32), j % (D / 32)); };
    f32x16 snext[BC / 32];
#pragma unroll
    for (int mt = 0; mt < BC / 32; ++mt) snext[mt] = (f32x16){};
    bf16x8 ka[NS], va[NP], pop[BC / 16];
    float lsum;
    u32x4 keepw[BC / 32];
    if constexpr (DROP) {
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt)
        keepw[mt] = dropout_bytes<false>(p.drop, bh, wq0, t * BC + 32 * mt, lane);
    }
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) ka[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + AHEAD < NS) ka[i + AHEAD] = kread(i + AHEAD);
      if (i >= NS - AHEAD) va[i - (NS - AHEAD)] = vread(i - (NS - AHEAD));
      snext[i / KS] = mfma32(ka[i], qop[i % KS], snext[i / KS]);
#pragma unroll
      for (int u = 0; u < EPB; ++u) {
        const int e = EPB * i + u, mt = e >> 4, r = e & 15;
        float x = fast_exp2(fmaf(scur[mt][r], s2, -mb));
        lsum = e == 0 ? x : lsum + x;  // (no 0 + x: an add the compiler must keep)
        if constexpr (DROP) x = dropout_keep(keepw[mt], r, p.drop.thresh) ? x : 0.f;
        pop[e >> 3][e & 7] = (__bf16)x;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float part[NCH];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j + AHEAD < NP) va[j + AHEAD] = vread(j + AHEAD);
      oacc[j % (D / 32)] = mfma32(va[j], pop[j / (D / 32)], oacc[j % (D / 32)]);
      if (j >= J0 && j - J0 < NCH) {
        const int c = j - J0;
        float mx = snext[(c * CH) >> 4][(c * CH) & 15];
#pragma unroll
        for (int u = 1; u < CH; ++u) {
          const int e = c * CH + u;
          if (e < NV) mx = fmaxf(mx, snext[e >> 4][e & 15]);
        }
        // Pin the slice here: it is only read after the loop, and the
        // compiler would otherwise sink it there, out of the bundles.
        asm volatile("" ::"v"(mx));
        part[c] = mx;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += lsum;
    if (t + 1 < t_hi) {
      float mx = part[0];
#pragma unroll
      for (int c = 1; c < NCH; ++c) mx = fmaxf(mx, part[c]);
      if (mask_tile(t + 1, snext)) mx = tile_max(snext);
      update_max(mx);
    }

    // The loads issued one iteration ago (K_{t+2}, V_{t+1}) have landed for
    // this wave; after the barrier they have for every wave, and the slots
    // read in this iteration may be refilled.  This iteration's loads stay
    // in flight.
    __builtin_amdgcn_s_waitcnt(kWaitOlderLoads);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int mt = 0; mt < BC / 32; ++mt) scur[mt] = snext[mt];
  };

  for (int t = t_lo; t < t_hi; t += 3) {
    iteration(t, sK1, sV0, sK0, sV2);
    if (t + 1 < t_hi) iteration(t + 1, sK2, sV1, sK1, sV0);
    if (t + 2 < t_hi) iteration(t + 2, sK0, sV2, sK2, sV1);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue: O = O~ / l, L = ln 2 * (m s2 + log2 l) ----
  const float l_tot = halves_sum(l_run);
  if (my_q < N) {
    const float inv = (DROP ? p.drop.inv_keep : 1.f) / l_tot;
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
          (m_run * s2 + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

// ------------------------------------------------------------- ping-pong
// Without dropout: the same computation in workgroups of 8 waves
// (256 queries), split into two groups (waves 0-3 and 4-7; the hardware
// places waves w and w + 4 on the same SIMD).  Each wave alternates a matrix
// half-step M(u) -- S of tile u+1 and O~ += P~_u V_u, 16 MFMAs and their
// operand reads -- with a vector half-step V(u) -- mask, row max, rescale and
// the exponentials of tile u+1 -- and the second group runs one half-step
// behind the first, so that on every SIMD one wave feeds the matrix cores
// while the other uses the VALU.  A barrier ends every half-step.  K_j and
// V_j sit in slot j % 3 of their rings; at every even half-step 2u the waves
// fetch K_{u+3} and V_{u+2}, and every half-step ends by waiting for the
// fetches issued two half-steps earlier, so that the operands of a wave's
// next M are in LDS during its V and the first of them are read there, at
// its start, before the exponentials (measured about 1 % faster than at its
// end).
// Under the causal mask the first group (the workgroup's first 128 queries)
// stops computing after the last tile its queries see and from then on only
// fetches its share of the tiles and joins the barriers.
// IN: 0 = bf16 inputs; 1 = e4m3 codes with one descale per tensor; 2 = e4m3
// codes with one descale per block.  With e4m3 inputs the products run on
// the 16-bit MFMAs, S = K Q^T in bf16 and O~ += V^T P^T in fp16, both of
// which hold every e4m3 value exactly.  The fp8 MFMA's sum of 64 products
// keeps too few bits below its largest product for the scores of inputs with
// outlier channels (their error then reaches the output amplified by the
// outlier channels of V), and an accurate fp8 P V needs P as two e4m3 terms,
// i.e. as many MFMA cycles as a 16-bit P V and more vector work.  P is fp16
// rather than bf16 because its rounding error reaches O multiplied by |V|,
// which the outlier channels make large.  Each K and V tile is copied to LDS
// as e4m3 (a staging ring of three slots) and widened there to the bf16 tile
// layout by one wave group during its matrix half-step, so that the rest of
// the kernel is the bf16 one.  The descales fold into the score scale and the
// output scale (per tensor), or into each tile's score scale and weights (per
// block; the weights then carry the value descale, which must stay below
// 2^8 so that they stay inside the fp16 range).
template <int D, int NG, int BC, int IN>
__device__ __forceinline__ void fwd_pp_body(const FwdKParams& p) {
  constexpr bool F8 = IN != 0, BLOCKS = IN == 2;
  constexpr int MT = BC / 32;          // score tiles of 32 keys per K/V tile
  constexpr int NWV = 2 * NG;          // waves
  constexpr int BR = 32 * NWV;         // queries per workgroup
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int AHEAD = 3;
  constexpr int NSM = MT * KS;         // S MFMAs of one M; as many P V MFMAs
  static_assert(NSM == (BC / 16) * DT, "S and P V products alternate one to one");
  __shared__ __attribute__((aligned(16))) __bf16 sK0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sK1[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sK2[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV1[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV2[BC * D];
  // e4m3 staging slots: the K tile, then the V tile, of one fetch.
  constexpr int SS = F8 ? 2 * BC * D : 16;
  __shared__ __attribute__((aligned(16))) uint8_t sS0[SS];
  __shared__ __attribute__((aligned(16))) uint8_t sS1[SS];
  __shared__ __attribute__((aligned(16))) uint8_t sS2[SS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const bool lead = w < NG;  // first group: M(u) at half-step 2u
  const int h = lane >> 5, n = lane & 31;
  const TileId id =
      tile_order(blockIdx.x, gridDim.x / p.n_qtiles, p.n_qtiles, p.causal, causal_group<D>());
  const int bh = id.bh;
  const int qt = p.causal ? p.n_qtiles - 1 - id.rank : id.rank;
  const int N = p.N;
  const int q0 = qt * BR;
  const int wq0 = q0 + 32 * w;
  const int my_q = wq0 + n;
  const size_t head = (size_t)bh * N * D;
  const size_t kv_off = (size_t)kv_head(bh, p.H, p.Hkv) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc(p.q + head, head_bytes);
  const __bf16* kh = p.k + kv_off;
  const __bf16* vh = p.v + kv_off;
  // e4m3 heads: one byte per element.
  const uint32_t head_bytes8 = (uint32_t)N * D;
  const uint8_t* kh8 = (const uint8_t*)p.k + kv_off;
  const uint8_t* vh8 = (const uint8_t*)p.v + kv_off;

  bf16x8 qop[KS];
  if constexpr (F8) {
    // Channels 16 ks + 8 h .. +7 of the query, widened.
    const auto rq8 = make_rsrc((const uint8_t*)p.q + head, head_bytes8);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 x = buf_load16(rq8, (uint32_t)(my_q * D + 16 * ks));
      qop[ks] = e4m3x8_to_bf16(h ? x[2] : x[0], h ? x[3] : x[1]);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = __builtin_bit_cast(
          bf16x8, buf_load16(rq, (uint32_t)(my_q * D + 16 * ks + 8 * h) * 2u));
  }

  const int q_last = min(q0 + BR, N) - 1;
  int kv_lo = 0, kv_hi = N;
  if (p.causal) kv_hi = min(kv_hi, q_last + 1);
  if (p.window > 0) {
    kv_lo = max(0, q0 - p.window + 1);
    if (!p.causal) kv_hi = min(kv_hi, q_last + p.window);
  }
  const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;
  const int T = t_hi - t_lo;

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = (f32x16){};
  float m_run = kMaxInit, l_run = 0.f;
  const float s2 = p.scale * kLog2e;
  const float tau = 8.0f / s2;
  const TrCoord trc(lane);
  // e4m3 inputs: the running max is kept in base-2 logit units (so that
  // tiles with different key descales compare directly).  A tile's code
  // products are scaled by s log2(e) dq dk (s2k with per-tensor descales,
  // s2q dk(tile) with block descales), and with block descales log2 of the
  // tile's value descale is folded into its weights.
  const int kvh = kv_head(bh, p.H, p.Hkv);
  const int n_kb = (N + 63) / 64;
  float s2q = 0.f, s2k = 0.f;
  if constexpr (F8) {
    s2q = s2 * (BLOCKS ? p.qs[(size_t)bh * ((N + 127) / 128) + (q0 + (lead ? 0 : 32 * NG)) / 128]
                       : p.q_descale);
    s2k = s2q * p.k_descale;
  }
  // Block descales: fetch(u) loads those of tile t_lo + u + 2 into set
  // u % 3, which V(u+1) reads.  They are read through the constant address
  // space, which makes them scalar loads (vector loads would join the
  // staging loads' in-order wait count); nothing writes them while the
  // kernel runs.
  typedef const __attribute__((address_space(4))) float* ConstF;
  float dks[3] = {1.f, 1.f, 1.f}, dvs[3] = {1.f, 1.f, 1.f};
  auto load_scales = [&](int t, int set) {
    if constexpr (BLOCKS) {
      const int i = kvh * n_kb + min(t * BC / 64, n_kb - 1);
      dks[set] = ((ConstF)p.ks)[i];
      dvs[set] = ((ConstF)p.vs)[i];
    }
  };

  int hi_key = N - 1, lo_key = 0;
  if (p.causal) hi_key = min(hi_key, my_q);
  if (p.window > 0) {
    lo_key = my_q - p.window + 1;
    if (!p.causal) hi_key = min(hi_key, my_q + p.window - 1);
  }
  // Masks tile t's scores when the tile straddles a boundary of this wave.
  auto mask_tile = [&](int t, f32x16* sacc) {
    const int kv0 = t * BC;
    bool need = kv0 + BC > N;
    if (p.causal) need |= kv0 + BC - 1 > wq0;
    if (p.window > 0) {
      need |= wq0 + 31 - kv0 >= p.window;
      if (!p.causal) need |= kv0 + BC - 1 - wq0 >= p.window;
    }
    if (!need) return;
    const int lim_hi = hi_key - kv0 - 4 * h, lim_lo = lo_key - kv0 - 4 * h;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * mt + 8 * (r >> 2) + (r & 3);
        sacc[mt][r] = (c > lim_hi || c < lim_lo) ? -__builtin_inff() : sacc[mt][r];
      }
  };

  // Byte offsets of this lane's operand reads in a tile (K rows per K-step;
  // V transposing reads per d-tile and row half), re-hidden from the
  // optimizer at every half-step so that slot constants fold into the reads.
  uint32_t roff[KS], toff[2 * DT];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = (uint32_t)tile_off<D>(n, 2 * ks + h) * 2u;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = trc.row + 8 * x, col = 32 * dt + trc.col;
      toff[2 * dt + x] = (uint32_t)(tile_off<D>(r, col >> 3) + (col & 7)) * 2u;
    }
  auto hide = [&]() {
#pragma unroll
    for (int i = 0; i < KS; ++i) asm volatile("" : "+v"(roff[i]));
#pragma unroll
    for (int i = 0; i < 2 * DT; ++i) asm volatile("" : "+v"(toff[i]));
  };
  // (Rows 32 mt + n share row n's swizzle, so a score tile mt is a constant
  // offset.)
  auto rrow = [&](const __bf16* t, int mt, int ks) {
    return *(const bf16x8*)((const char*)t + roff[ks] + mt * 32 * D * 2);
  };
  auto rtr = [&](const __bf16* t, int j) {  // K-step j / DT, d-tile j % DT
    const char* b = (const char*)t + 16 * (j / DT) * D * 2;
    return cat4(lds_read_tr16(b + toff[2 * (j % DT)]), lds_read_tr16(b + toff[2 * (j % DT) + 1]));
  };

  f32x16 snx[MT];  // raw scores of the tile whose probabilities come next
  bf16x8 pop[BC / 16];
  // Row max of snx (masked), running max moved past it, O~ and l rescaled,
  // then the probabilities of snx into pop and their sum into l.
  // set: the descale set holding this tile's block descales.
  // Block descales: the score scale, log2 of the value descale and its
  // inverse for the next softmax step, formed from descale set `set` during
  // the matrix half-step before it (where the vector units have time).
  float tsc = 0.f, tlv = 0.f, trl = 1.f;
  auto tile_consts = [&](int set) {
    if constexpr (BLOCKS) {
      tsc = s2q * dks[set];
      tlv = __builtin_amdgcn_logf(dvs[set]);
      trl = fast_exp2(-tlv);
    }
  };
  auto softmax_step_f8 = [&]() {
    float mx = snx[0][0];
#pragma unroll
    for (int e = 1; e < 16 * MT; ++e) mx = fmaxf(mx, snx[e >> 4][e & 15]);
    const float sc = BLOCKS ? tsc : s2k, lvt = BLOCKS ? tlv : 0.f;
    mx = halves_max(mx) * sc;
    const float m_new = (mx > m_run + 8.f) ? mx : m_run;
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    const float mb = m_run - lvt;
    float lsum;
#pragma unroll
    for (int e = 0; e < 16 * MT; e += 2) {  // fp16 weights, two per convert
      const float x0 = fast_exp2(fmaf(snx[e >> 4][e & 15], sc, -mb));
      const float x1 = fast_exp2(fmaf(snx[e >> 4][(e & 15) + 1], sc, -mb));
      lsum = e == 0 ? x0 + x1 : lsum + x0 + x1;
      const auto hb = __builtin_bit_cast(bf16x2, (f16x2){(_Float16)x0, (_Float16)x1});
      pop[e >> 3][e & 7] = hb[0];
      pop[e >> 3][(e & 7) + 1] = hb[1];
    }
    // The weights carry the value descale; l sums them without it.
    l_run += BLOCKS ? lsum * trl : lsum;
  };
  auto softmax_step = [&]() {
    float mx = snx[0][0];
#pragma unroll
    for (int e = 1; e < 16 * MT; ++e) mx = fmaxf(mx, snx[e >> 4][e & 15]);
    mx = halves_max(mx);
    const float m_new = (mx > m_run + tau) ? mx : m_run;
    const float alpha = fast_exp2((m_run - m_new) * s2);
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    const float mb = m_run * s2;
    float lsum;
#pragma unroll
    for (int e = 0; e < 16 * MT; ++e) {
      const float x = fast_exp2(fmaf(snx[e >> 4][e & 15], s2, -mb));
      lsum = e == 0 ? x : lsum + x;
      pop[e >> 3][e & 7] = (__bf16)x;
    }
    l_run += lsum;
  };

  // e4m3 tiles: the first group stages and widens the K tiles, the second
  // the V tiles; each lane widens one 16-byte chunk (16 codes) of a tile.
  const int wg = lead ? w : w - NG;  // wave index inside its group
  static_assert(!F8 || (BC * D / 16 == 64 * NG && 32 * NG == 128), "e4m3 tile split");
  const int wpc = wg * 64 + lane;  // the chunk this lane widens
  const int wrow = wpc / (D / 16), wch = 2 * (wpc % (D / 16));
  // Which of its two bf16 chunks a lane stores (and reads) first.  The LDS
  // serves 8 lanes of a 16-byte store per cycle; they must hit 8 different
  // 16-byte bank slots modulo 128 bytes, i.e. different chunk indices mod 8
  // (the swizzle XOR keeps them so).  At d = 128 those 8 lanes are the 8
  // chunks of one row: the first half stores its even chunks, the second its
  // odd ones.  At d = 64 they are two rows: one stores even chunks, the other
  // odd (their swizzles have the same parity).  The order also alternates
  // between the rows whose 8-byte reads meet in one cycle.  (Measured: 16 %
  // of the LDS cycles were bank conflicts with one order for all lanes.)
  const int wodd = D == 128 ? (((wpc % 8) >> 2) ^ wrow) & 1 : (wrow ^ (wrow >> 1)) & 1;
  const int woff0 = tile_off<D>(wrow, wch + wodd), woff1 = tile_off<D>(wrow, wch + 1 - wodd);
  // The lane's 16 codes, the half stored first in x[0..1].
  auto wread = [&](const uint8_t* chunk) {
    const u32x2 a = *(const u32x2*)&chunk[8 * wodd], b = *(const u32x2*)&chunk[8 - 8 * wodd];
    return (u32x4){a[0], a[1], b[0], b[1]};
  };
  auto stage = [&](int t, uint8_t* slot) {  // this group's tile t into a staging slot
    if (lead) tile_stage_lds8<D, BC, NG>(kh8, head_bytes8, t * BC, slot, wg, lane);
    else tile_stage_lds8<D, BC, NG>(vh8, head_bytes8, t * BC, slot + BC * D, wg, lane);
  };
  // K is widened to bf16, V to fp16 (stored in the same 16-bit tile layout).
  auto widen8 = [&](uint32_t x0, uint32_t x1) {
    return lead ? e4m3x8_to_bf16(x0, x1) : __builtin_bit_cast(bf16x8, e4m3x8_to_f16(x0, x1));
  };
  auto widen = [&](const uint8_t* slot, __bf16* dst) {  // this group's half of a slot
    const u32x4 x = wread(&slot[(lead ? 0 : BC * D) + wpc * 16]);
    *(bf16x8*)&dst[woff0] = widen8(x[0], x[1]);
    *(bf16x8*)&dst[woff1] = widen8(x[2], x[3]);
  };

  // Prologue: K_0, K_1, K_2, V_0, V_1 (tile j = t_lo + j); S of tile 0 and
  // its probabilities.  e4m3: K_0, K_1, V_0, V_1 staged and widened here (K_1
  // staged in K_2's bf16 slot, which is free until K_2 is widened), K_2 and
  // V_1 staged in slot 1, K_3 and V_2 in slot 2.
  if constexpr (F8) {
    stage(t_lo, sS0);
    load_scales(t_lo, 0);
    load_scales(t_lo + 1, 2);
    if (lead) stage(t_lo + 1, (uint8_t*)sK2);
    stage(t_lo + 2, lead ? sS1 : sS2);  // K_2 / V_2
    stage(t_lo + (lead ? 3 : 1), lead ? sS2 : sS1);  // K_3 / V_1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    widen(sS0, lead ? sK0 : sV0);
    if (lead) {
      const u32x4 x = wread(&((const uint8_t*)sK2)[wpc * 16]);
      *(bf16x8*)&sK1[woff0] = e4m3x8_to_bf16(x[0], x[1]);
      *(bf16x8*)&sK1[woff1] = e4m3x8_to_bf16(x[2], x[3]);
    } else {
      widen(sS1, sV1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  } else {
    tile_load_lds<D, BC, NWV>(kh, head_bytes, t_lo * BC, sK0, w, lane);
    tile_load_lds<D, BC, NWV>(vh, head_bytes, t_lo * BC, sV0, w, lane);
    tile_load_lds<D, BC, NWV>(kh, head_bytes, (t_lo + 1) * BC, sK1, w, lane);
    tile_load_lds<D, BC, NWV>(vh, head_bytes, (t_lo + 1) * BC, sV1, w, lane);
    tile_load_lds<D, BC, NWV>(kh, head_bytes, (t_lo + 2) * BC, sK2, w, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    snx[mt] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      snx[mt] = mfma32(tile_row8<D>(sK0, 32 * mt + n, 2 * ks + h), qop[ks], snx[mt]);
  }
  mask_tile(t_lo, snx);
  if constexpr (F8) {
    tile_consts(0);
    softmax_step_f8();
  } else {
    softmax_step();
  }
  __syncthreads();  // every wave has read K_0 before its slot is refilled

  // Half-step end: the wait for the fetches issued two half-steps earlier
  // (this wave's two latest stay in flight), then the barrier; so the tiles
  // that M(u+1) reads are in LDS for every wave from the half-step before it.
  // e4m3: one staging load per wave and fetch, so the wait leaves that one
  // in flight, and the widening stores must be done before the barrier.
  auto end_half = [&]() {
    if constexpr (F8) __builtin_amdgcn_s_waitcnt(waitcnt_vm(1) & ~(0xF << 8));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(2));
    __builtin_amdgcn_s_barrier();
  };
  // Fetches of even half-step 2u: K_{u+3} into K_u's slot, V_{u+2} into V_{u-1}'s.
  // e4m3: K_{u+4} and V_{u+3} into staging slot u % 3 (Kf: that slot; Vf
  // unused); the first group widens K_{u+2} during M(u) (half-step 2u), the
  // second V_{u+2} during M(u) (half-step 2u + 1), each from the slot that
  // fetch(u-2) or fetch(u-1) filled.
  auto fetch = [&](int u, auto* Kf, auto* Vf) {
    if constexpr (F8) {
      (void)Vf;
      stage(t_lo + u + (lead ? 4 : 3), (uint8_t*)Kf);
      // (Kf is staging slot u % 3, and so names the descale set.)
      load_scales(t_lo + u + 2, (uint8_t*)Kf == sS0 ? 0 : (uint8_t*)Kf == sS1 ? 1 : 2);
    } else {
      tile_load_lds<D, BC, NWV>(kh, head_bytes, (t_lo + u + 3) * BC, Kf, w, lane);
      tile_load_lds<D, BC, NWV>(vh, head_bytes, (t_lo + u + 2) * BC, Vf, w, lane);
    }
  };
  // M(u): S of tile u+1 from Kn (into snx) and O~ += V_u^T P~_u^T from Vc,
  // the two kinds of MFMA alternating; operand i is read AHEAD MFMAs before
  // its use, the first AHEAD by prefetch() in the half-step before.
  bf16x8 ka[NSM], va[NSM];
  auto issue = [&](int i, const __bf16* Kn, const __bf16* Vc) {
    if (i & 1) va[i >> 1] = rtr(Vc, i >> 1);
    else ka[i >> 1] = rrow(Kn, (i >> 1) / KS, (i >> 1) % KS);
  };
  auto prefetch = [&](const __bf16* Kn, const __bf16* Vc) {
    hide();
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) issue(i, Kn, Vc);
  };
  // Wsrc, Wdst (e4m3): the staging slot and bf16 slot of this group's
  // widening, spread over three of the half-step's MFMAs.
  // vset: the descale set of V(u)'s tile, t_lo + u + 1, which fetch(u-1)
  // filled: (u + 2) % 3 (a constant at every call).
  auto mstep = [&](const __bf16* Kn, const __bf16* Vc, const uint8_t* Wsrc = nullptr,
                   __bf16* Wdst = nullptr, int vset = 0) {
    tile_consts(vset);
    hide();
    f32x16 s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s[mt] = (f32x16){};
    u32x4 wx;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * NSM; ++i) {
      if (i + AHEAD < 2 * NSM) issue(i + AHEAD, Kn, Vc);
      if constexpr (F8) {
        if (i == 2) wx = wread(&Wsrc[(lead ? 0 : BC * D) + wpc * 16]);
        if (i == 6) *(bf16x8*)&Wdst[woff0] = widen8(wx[0], wx[1]);
        if (i == 10) *(bf16x8*)&Wdst[woff1] = widen8(wx[2], wx[3]);
      }
      if (i & 1) {
        const int j = i >> 1;
        if constexpr (F8)
          oacc[j % DT] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8, va[j]), __builtin_bit_cast(f16x8, pop[j / DT]),
              oacc[j % DT], 0, 0, 0);
        else
          oacc[j % DT] = mfma32(va[j], pop[j / DT], oacc[j % DT]);
      } else {
        const int si = i >> 1;
        s[si / KS] = mfma32(ka[si], qop[si % KS], s[si / KS]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) snx[mt] = s[mt];
  };
  // V(u): probabilities of tile u+1 (when this group computes one; V(-1) of
  // the second group is the prologue's).
  auto vstep = [&](int u, int Tg) {
    if (u >= 0 && u + 1 < Tg) {
      mask_tile(t_lo + u + 1, snx);
      if constexpr (F8) softmax_step_f8();
      else softmax_step();
    }
  };

  // Half-steps 0 .. 2T: the lead group runs M(u) at 2u and V(u) at 2u+1,
  // the other V(u-1) at 2u and M(u) at 2u+1; both end with one more.  (The
  // operands prefetched after a group's last M are read but never used.)
  int u = 0;
  if (lead) {
    // With the causal mask the first group's queries (the workgroup's first
    // 32 * NG) see only the tiles up to theirs; it computes those and then
    // only fetches its share of the later tiles and joins the barriers.
    const int Tg = p.causal ? min(T, (q0 + 32 * NG - 1) / BC - t_lo + 1) : T;
    prefetch(sK1, sV0);
    for (; u + 3 <= Tg; u += 3) {
      if constexpr (F8) fetch(u, sS0, sV2), mstep(sK1, sV0, sS1, sK2, 2);
      else fetch(u, sK0, sV2), mstep(sK1, sV0);
      end_half();
      prefetch(sK2, sV1);
      vstep(u, Tg);
      end_half();
      if constexpr (F8) fetch(u + 1, sS1, sV0), mstep(sK2, sV1, sS2, sK0, 0);
      else fetch(u + 1, sK1, sV0), mstep(sK2, sV1);
      end_half();
      prefetch(sK0, sV2);
      vstep(u + 1, Tg);
      end_half();
      if constexpr (F8) fetch(u + 2, sS2, sV1), mstep(sK0, sV2, sS0, sK1, 1);
      else fetch(u + 2, sK2, sV1), mstep(sK0, sV2);
      end_half();
      prefetch(sK1, sV0);
      vstep(u + 2, Tg);
      end_half();
    }
    if (u < Tg) {
      if constexpr (F8) fetch(u, sS0, sV2), mstep(sK1, sV0, sS1, sK2, 2);
      else fetch(u, sK0, sV2), mstep(sK1, sV0);
      end_half();
      prefetch(sK2, sV1);
      vstep(u, Tg);
      end_half();
    }
    if (u + 1 < Tg) {
      if constexpr (F8) fetch(u + 1, sS1, sV0), mstep(sK2, sV1, sS2, sK0, 0);
      else fetch(u + 1, sK1, sV0), mstep(sK2, sV1);
      end_half();
      prefetch(sK0, sV2);
      vstep(u + 1, Tg);
      end_half();
    }
    for (u += (u < Tg) + (u + 1 < Tg); u < T; ++u) {
      if constexpr (F8) {
        // Still widens the K tiles that the other group reads.
        // (Widening first: its reads then follow no pending copy.)
        if (u % 3 == 0) widen(sS1, sK2), fetch(u, sS0, sV2);
        else if (u % 3 == 1) widen(sS2, sK0), fetch(u, sS1, sV0);
        else widen(sS0, sK1), fetch(u, sS2, sV1);
      } else {
        if (u % 3 == 0) fetch(u, sK0, sV2);
        else if (u % 3 == 1) fetch(u, sK1, sV0);
        else fetch(u, sK2, sV1);
      }
      end_half();
      end_half();
    }
    end_half();
  } else {
    for (; u + 3 <= T; u += 3) {
      if constexpr (F8) fetch(u, sS0, sV2);
      else fetch(u, sK0, sV2);
      prefetch(sK1, sV0);
      vstep(u - 1, T);
      end_half();
      if constexpr (F8) mstep(sK1, sV0, sS2, sV2, 2);
      else mstep(sK1, sV0);
      end_half();
      if constexpr (F8) fetch(u + 1, sS1, sV0);
      else fetch(u + 1, sK1, sV0);
      prefetch(sK2, sV1);
      vstep(u, T);
      end_half();
      if constexpr (F8) mstep(sK2, sV1, sS0, sV0, 0);
      else mstep(sK2, sV1);
      end_half();
      if constexpr (F8) fetch(u + 2, sS2, sV1);
      else fetch(u + 2, sK2, sV1);
      prefetch(sK0, sV2);
      vstep(u + 1, T);
      end_half();
      if constexpr (F8) mstep(sK0, sV2, sS1, sV1, 1);
      else mstep(sK0, sV2);
      end_half();
    }
    if (u < T) {
      if constexpr (F8) fetch(u, sS0, sV2);
      else fetch(u, sK0, sV2);
      prefetch(sK1, sV0);
      vstep(u - 1, T);
      end_half();
      if constexpr (F8) mstep(sK1, sV0, sS2, sV2, 2);
      else mstep(sK1, sV0);
      end_half();
    }
    if (u + 1 < T) {
      if constexpr (F8) fetch(u + 1, sS1, sV0);
      else fetch(u + 1, sK1, sV0);
      prefetch(sK2, sV1);
      vstep(u, T);
      end_half();
      if constexpr (F8) mstep(sK2, sV1, sS0, sV0, 0);
      else mstep(sK2, sV1);
      end_half();
    }
    end_half();
  }
  __builtin_amdgcn_s_waitcnt(0);  // no fetch may land after the workgroup ends

  const float l_tot = halves_sum(l_run);
  if (my_q < N) {
    const float inv = (IN == 1 ? p.v_descale : 1.f) / l_tot;
    const size_t row = head + (size_t)my_q * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
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
          ((F8 ? m_run : m_run * s2) + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

template <int D, int NG, int BC>
__global__ __launch_bounds__(2 * NG * 64, 2) void fwd_pp_kernel(FwdKParams p) {
  fwd_pp_body<D, NG, BC, 0>(p);
}
template <int D, int NG, int BC, bool BLOCKS>
__global__ __launch_bounds__(2 * NG * 64, 2) void fwd_fp8_pp_kernel(FwdKParams p) {
  fwd_pp_body<D, NG, BC, BLOCKS ? 2 : 1>(p);
}

// Kernel parameters for workgroups of `rows` queries.
static FwdKParams fwd_params(const FwdArgs& a, int rows) {
  FwdKParams p;
  p.q = (const __bf16*)a.q;
  p.k = (const __bf16*)a.k;
  p.v = (const __bf16*)a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.H = a.H;
  p.Hkv = a.Hkv;
  p.N = a.N;
  p.n_qtiles = (a.N + rows - 1) / rows;
  p.scale = a.scale;
  p.causal = a.causal;
  p.window = a.window;
  p.out_f32 = a.out_f32;
  p.drop = make_dropout(a.drop);
  p.q_descale = p.k_descale = p.v_descale = 1.f;
  p.qs = p.ks = p.vs = nullptr;
  return p;
}

template <int D, int NW, int BC, bool DROP>
static hipError_t launch_fwd_cfg(const FwdArgs& a, hipStream_t stream, const char** name) {
  const FwdKParams p = fwd_params(a, 32 * NW);
  const unsigned grid = (unsigned)(a.BH * p.n_qtiles);
  return go<fwd_bf16_kernel<D, NW, BC, DROP>>(name, kname("attn::fwd_bf16_kernel", D, NW, BC, DROP),
                                              dim3(grid), dim3(NW * 64), stream, p);
}

// Without dropout: the ping-pong kernel (two groups of 4 waves), 32-key tiles
// at d = 128 and 64-key tiles at d = 64.
template <int D, int BC>
static hipError_t launch_fwd_pp(const FwdArgs& a, hipStream_t stream, const char** name) {
  constexpr int NG = 4;
  const FwdKParams p = fwd_params(a, 64 * NG);
  return go<fwd_pp_kernel<D, NG, BC>>(name, kname("attn::fwd_pp_kernel", D, NG, BC),
                                      dim3((unsigned)(a.BH * p.n_qtiles)), dim3(2 * NG * 64),
                                      stream, p);
}

// e4m3 inputs on the ping-pong kernel (same tiles as bf16).
template <int D, int BC>
static hipError_t launch_fwd_fp8_d(const FwdArgs& a, hipStream_t stream, const char** name) {
  constexpr int NG = 4;
  FwdKParams p = fwd_params(a, 64 * NG);
  p.q_descale = a.q_descale;
  p.k_descale = a.k_descale;
  p.v_descale = a.v_descale;
  p.qs = a.q_scales;
  p.ks = a.k_scales;
  p.vs = a.v_scales;
  const dim3 grid((unsigned)(a.BH * p.n_qtiles)), block(2 * NG * 64);
  if (a.q_scales)
    return go<fwd_fp8_pp_kernel<D, NG, BC, true>>(
        name, kname("attn::fwd_fp8_pp_kernel", D, NG, BC, true), grid, block, stream, p);
  return go<fwd_fp8_pp_kernel<D, NG, BC, false>>(
      name, kname("attn::fwd_fp8_pp_kernel", D, NG, BC, false), grid, block, stream, p);
}

hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream, const char** name) {
  if (a.d == 128) return launch_fwd_fp8_d<128, 32>(a, stream, name);
  return launch_fwd_fp8_d<64, 64>(a, stream, name);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream, const char** name) {
  if (a.drop.thresh > 0) {
    if (a.d == 128) return launch_fwd_cfg<128, 4, 32, true>(a, stream, name);
    return launch_fwd_cfg<64, 4, 64, true>(a, stream, name);
  }
  // Grids of fewer than four 256-query workgroups (one short head, say):
  // 128-query workgroups give twice the parallelism, and such a launch is
  // bound by latency, not by the matrix cores.
  if (a.BH * ((a.N + 255) / 256) < 4) {
    if (a.d == 128) return launch_fwd_cfg<128, 4, 32, false>(a, stream, name);
    return launch_fwd_cfg<64, 4, 64, false>(a, stream, name);
  }
  if (a.d == 128) return launch_fwd_pp<128, 32>(a, stream, name);
  return launch_fwd_pp<64, 64>(a, stream, name);
}

}  // namespace attn

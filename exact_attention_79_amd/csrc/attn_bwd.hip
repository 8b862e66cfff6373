// attn_bwd.hip -- bf16 backward kernels for gfx950.
//
// Method (FLASH-ATTN page, FlashAttention-2 summary, "Background": dV = P^T dO,
// dP = dO V^T, dS = dsoftmax(dP), dQ = dS K, dK = dS^T Q).  P is recomputed
// tile by tile from Q, K and the forward's log-sum-exp L (the "Tiling and
// Recomputation" section: only the softmax statistics are kept from the
// forward), as P_ij = exp(s S_ij - L_i).  The softmax Jacobian is applied as
// dS_ij = P_ij (dP_ij - D_i) with D_i = sum_k dO_ik O_ik, and the scale s of
// S = s Q K^T gives dQ = s dS K and dK = s dS^T Q.
//
// Two launches on the caller's stream (which kernel serves which head dim
// and mask: without dropout, bwd_dq_pp_kernel at d = 128, bwd_dkdv_quad_kernel
// at d = 128 and bwd_dkdv_pp_kernel at d = 64 non-causal; the single-wave
// kernels otherwise):
//  1. bwd_dq_kernel: one workgroup per query block, Q_i, dO_i, L_i, D_i
//     resident, looping over the K/V blocks it sees; dQ_i accumulates in
//     VGPRs and is written once.  Each lane owns one query row, so it forms
//     D_i = rowsum(dO_i * O_i) itself (one read of O_i) and also leaves D_i
//     and L_i log2(e) in the workspace for the second launch;
//  2. bwd_dkdv_kernel: one workgroup per K/V block (the page's column-block
//     partition of the backward), K_j and V_j resident in VGPRs, looping over
//     the query blocks that can see them; dK_j and dV_j accumulate in VGPRs
//     and are written once.
// bwd_delta_kernel writes the same two workspace arrays on its own (for
// callers that run the dK/dV pass without the dQ pass).
// Splitting dQ into its own pass recomputes S and dP there (two extra
// products per visible tile) but needs no atomics and no zeroed buffer, and
// the result is deterministic.
//
// gfx950 mapping.  In the dK/dV kernels a wave owns 32 keys (64 in the
// four-role kernel) and computes S = Q K^T with keys on the MFMA N side, so
// the C layout gives one key per lane and P, dS (bf16) are directly the B
// operands of dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T are read from
// LDS with transposing reads in the C layout's row permutation.  The dQ
// kernel is the mirror image: S^T = K Q^T with one query per lane, and
// dQ^T += K^T dS^T with K^T read transposed from LDS.  Q/dO (dK/dV kernels)
// and K/V (dQ kernel) tiles stream through LDS rings (direct global -> LDS
// loads) with the same swizzle as the forward.
#include <limits.h>

#include <algorithm>
#include <type_traits>

#include "attn_device.hpp"
#include "attn_kernels.hpp"

namespace attn {

__device__ __forceinline__ float bf16_lo(uint32_t x) {
  return __builtin_bit_cast(float, x << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t x) {
  return __builtin_bit_cast(float, x & 0xffff0000u);
}

// D_i = sum_k dO_ik O_ik over rows of d elements (D/8 threads per row), and
// L_i log2(e), the base-2 form of the log-sum-exp the other kernels use.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const __bf16* o,
                                                        const __bf16* dout,
                                                        const float* lse, float* delta,
                                                        float* lse2, int rows) {
  constexpr int TPR = D / 8;
  const int tid = threadIdx.x;
  const int r = blockIdx.x * (256 / TPR) + tid / TPR;
  const int c = tid % TPR;
  float acc = 0.f;
  if (r < rows) {
    const u32x4 a = *(const u32x4*)(o + (size_t)r * D + c * 8);
    const u32x4 b = *(const u32x4*)(dout + (size_t)r * D + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc += bf16_lo(a[i]) * bf16_lo(b[i]) + bf16_hi(a[i]) * bf16_hi(b[i]);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (r < rows && c == 0) {
    delta[r] = acc;
    lse2[r] = lse[r] * kLog2e;
  }
}

struct BwdKParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;  // natural-log L from the forward (dQ kernel)
  float* delta;      // workspace: D_i
  float* lse2;       // workspace: L_i log2(e)
  float* dk_part;    // workspace: partial dK, dV of each share (split > 1)
  float* dv_part;
  int split;         // workgroups per key block and group (dkdv_split)
  int H, Hkv;        // query heads per batch element; key/value heads
  float* dq;
  float* dk;
  float* dv;
  int N;
  int n_tiles;
  float scale;
  int causal, window;
  Dropout drop;
};

// ---------------------------------------------------------------- dK, dV
// Waves per SIMD of the dK/dV kernel: one (512 registers) in general; at
// d = 64 with 32-row query steps a wave fits in 256, and a second wave per
// SIMD overlaps one wave's exponentials with the other's MFMAs (measured
// 17-22 % faster than one wave with 64-row steps).
template <int D, int BQ>
constexpr int dkdv_waves_per_simd() { return (D == 64 && BQ == 32) ? 2 : 1; }

// One workgroup per block of 32*NW keys of one key/value head; wave w owns
// keys kw0 .. kw0+31 (one per lane on the MFMA N side).  Query tiles of BQ
// rows stream through three LDS slots (Q, dO and their L, D) fetched one
// tile ahead by direct global->LDS loads: the visible tiles of the first
// query head that reads this key/value head, then those of the next one of
// its group, and so on, so that dK and dV are summed over the group in
// registers (the FLASH-ATTN page's MQA/GQA paragraph).  Iteration i computes
// S and dP for tile i+1 on the matrix cores while the VALU forms P and dS
// for tile i, then accumulates dV += P^T dO and dK += dS^T Q for tile i.
// DROP: dropout on P with the forward's keep bytes: dV takes the kept P (its
// 1 / keep scale applied once at the end) and dS = P (Z dP / keep - D).
template <int D, int NW, int BQ, bool DROP>
__global__ __launch_bounds__(NW * 64, (dkdv_waves_per_simd<D, BQ>())) void bwd_dkdv_kernel(
    BwdKParams p) {
  constexpr int BKV = 32 * NW;
  constexpr int KS = D / 16;
  static_assert(BQ == 32 || BQ == 64, "query tile");
  constexpr int LDROWS = 64;  // L and D are staged one dword per lane of a wave
  __shared__ __attribute__((aligned(16))) __bf16 sQ0[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ1[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ2[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO0[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO1[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO2[BQ * D];
  __shared__ __attribute__((aligned(16))) float sL0[LDROWS], sL1[LDROWS], sL2[LDROWS];
  __shared__ __attribute__((aligned(16))) float sD0[LDROWS], sD1[LDROWS], sD2[LDROWS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int h = lane >> 5, n = lane & 31;
  // Low key blocks see the most queries under the causal mask: rank = block.
  // The grid's heads are (key/value head, share) pairs, the shares of one
  // key/value head adjacent (same XCD, same K and V).
  const TileId id =
      tile_order(blockIdx.x, gridDim.x / p.n_tiles, p.n_tiles, p.causal, causal_group<D>());
  const int bkv = id.bh / p.split;   // key/value head (b * Hkv + hk)
  const int share = id.bh % p.split;
  const int kt = id.rank;
  const int N = p.N, W = p.window;
  const int G = p.H / p.Hkv / p.split;  // query heads this workgroup walks
  const int bh0 = (bkv / p.Hkv) * p.H + (bkv % p.Hkv) * (p.H / p.Hkv) + share * G;
  const int k0 = kt * BKV;
  const int kw0 = k0 + 32 * w;
  const int my_k = kw0 + n;
  const size_t head = (size_t)bkv * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rk = make_rsrc(p.k + head, head_bytes);
  const auto rv = make_rsrc(p.v + head, head_bytes);

  // K^T and V^T as B operands (lane = key, 8 consecutive d per K-step).
  bf16x8 kop[KS], vop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)(my_k * D + 16 * ks + 8 * h) * 2u;
    kop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
    vop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
  }
  // Without dropout the dP MFMAs start from D_i and take -V, so that they
  // leave D_i - dP_ij: the subtraction of dsoftmax costs no vector
  // instruction, and the dS they give is negated, which the scale applied
  // to dK at the end undoes.  (With dropout, dP is scaled by the keep mask
  // before D is subtracted.)
  if constexpr (!DROP) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      vop[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vop[ks]) ^ 0x80008000u);
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dkacc[dt] = dvacc[dt] = (f32x16){};

  // Queries that can see any key of this block, and those that see my_k.
  const int k_last = min(k0 + BKV, N) - 1;
  int q_lo = p.causal ? k0 : 0, q_hi = N;
  int qmin = p.causal ? my_k : INT_MIN, qmax = INT_MAX;
  if (W > 0) {
    q_lo = max(q_lo, k0 - W + 1);
    q_hi = min(q_hi, k_last + W);
    if (!p.causal) qmin = my_k - W + 1;
    qmax = my_k + W - 1;
  }
  const int t_lo = q_lo / BQ, t_hi = (q_hi + BQ - 1) / BQ;

  const float s2 = p.scale * kLog2e;
  const TrCoord trc(lane);

  // Tiles are taken in the order (query head j of the group, tile t): the
  // load cursor (lj, lt) runs two tiles ahead of the compute cursor ct.
  // Past the last head it keeps reading the last head's rows (in bounds;
  // those tiles are never used).
  int lj = 0, lt = t_lo, ct = t_lo, cj = 0;
  auto load_tile = [&](__bf16* Qf, __bf16* Of, float* Lf, float* Df) {
    const int bhq = bh0 + min(lj, G - 1);
    const size_t qhead = (size_t)bhq * N * D;
    tile_load_lds<D, BQ, NW>(p.q + qhead, head_bytes, lt * BQ, Qf, w, lane);
    tile_load_lds<D, BQ, NW>(p.dout + qhead, head_bytes, lt * BQ, Of, w, lane);
    if (w == 0) {
      vec_load_lds<LDROWS>(make_rsrc(p.lse2 + (size_t)bhq * N, (uint32_t)N * 4), lt * BQ,
                           Lf, lane);
      vec_load_lds<LDROWS>(make_rsrc(p.delta + (size_t)bhq * N, (uint32_t)N * 4), lt * BQ,
                           Df, lane);
    }
    if (++lt == t_hi) {
      lt = t_lo;
      ++lj;
    }
  };
  // Start of the dP accumulator of M-tile mt: zero with dropout, else D of
  // the query rows this lane holds there (C layout: register 4g + c is row
  // 32 mt + 8 g + 4 h + c).
  auto dp_init = [&](const float* Ds, int mt) {
    f32x16 c = {};
    if constexpr (!DROP) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = *(const f32x4*)&Ds[32 * mt + 8 * g + 4 * h];
#pragma unroll
        for (int i = 0; i < 4; ++i) c[4 * g + i] = v[i];
      }
    }
    return c;
  };
  // S = Q K^T and dP = dO V^T (without dropout D - dP) for one tile
  // (queries on M, this wave's keys on N).
  auto sdp = [&](const __bf16* Qs, const __bf16* Os, const float* Ds, f32x16* sacc,
                 f32x16* dpacc) {
#pragma unroll
    for (int mt = 0; mt < BQ / 32; ++mt) {
      sacc[mt] = (f32x16){};
      dpacc[mt] = dp_init(Ds, mt);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sacc[mt] = mfma32(tile_row8<D>(Qs, 32 * mt + n, 2 * ks + h), kop[ks], sacc[mt]);
        dpacc[mt] = mfma32(tile_row8<D>(Os, 32 * mt + n, 2 * ks + h), vop[ks], dpacc[mt]);
      }
    }
  };

  // Prologue: tiles t_lo and t_lo+1; S, dP of the first tile.  Tiles past
  // the last visible one read as zeros (rows >= N) or are never used.
  load_tile(sQ0, sO0, sL0, sD0);
  load_tile(sQ1, sO1, sL1, sD1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 scur[BQ / 32], dpcur[BQ / 32];
  sdp(sQ0, sO0, sD0, scur, dpcur);

  // Iteration for the tile u of the sequence (query tile ct): P, dS of tile
  // u (slot c: Qc, Oc, Lc, Dc) while S, dP of tile u+1 (slot n: Qn, On, Dn)
  // run on the matrix cores; tile u+2 is fetched into slot f (tile u-1's,
  // fully consumed).
  auto iteration = [&](const __bf16* Qc, const __bf16* Oc, const float* Lc,
                       const float* Dc, const __bf16* Qn, const __bf16* On,
                       const float* Dn, __bf16* Qf, __bf16* Of, float* Lf, float* Df) {
    load_tile(Qf, Of, Lf, Df);
    const int i0 = ct * BQ;
    const int bhq = bh0 + cj;  // query head of this tile
    if (++ct == t_hi) {
      ct = t_lo;
      ++cj;
    }
    u32x4 keepw[BQ / 32];
    if constexpr (DROP) {
#pragma unroll
      for (int mt = 0; mt < BQ / 32; ++mt)
        keepw[mt] = dropout_bytes<true>(p.drop, bhq, i0 + 32 * mt, kw0, lane);
    }
    bool need_mask = false;
    if (p.causal) need_mask |= i0 < kw0 + 31;
    if (W > 0) {
      need_mask |= (i0 + BQ - 1) - kw0 >= W;
      if (!p.causal) need_mask |= (kw0 + 31) - i0 >= W;
    }
    if (need_mask) {
#pragma unroll
      for (int mt = 0; mt < BQ / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = i0 + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
          scur[mt][r] = (q < qmin || q > qmax) ? -__builtin_inff() : scur[mt][r];
        }
    }
    // L log2(e) and D of the query rows this lane holds, four rows (one
    // group g) at a time: group g covers rows 32 (g / 4) + 8 (g % 4) + 4h +
    // 0..3.  They are read two groups before use, so that waiting for them
    // never drains the operand reads queued behind them.
    auto lrow = [&](int g) { return *(const f32x4*)&Lc[32 * (g >> 2) + 8 * (g & 3) + 4 * h]; };
    auto drow = [&](int g) { return *(const f32x4*)&Dc[32 * (g >> 2) + 8 * (g & 3) + 4 * h]; };
    f32x4 lb[BQ / 8], dl[BQ / 8];

    constexpr int NS = 2 * (BQ / 32) * KS;     // S and dP MFMAs of the next tile
    constexpr int NP = 2 * (BQ / 16) * (D / 32);  // dV and dK MFMAs of this tile
    constexpr int EPB = (BQ / 2) / NS;        // P/dS elements per lane per bundle
    constexpr int AHEAD = 3;
    static_assert(EPB >= 1 && (BQ / 2) % NS == 0, "bundle split");
    // Score bundle i: MFMA (i even: S, odd: dP) of M-tile mt, K-step ks.
    auto arow = [&](int i) {
      const int j = i >> 1, mt = j / KS, ks = j % KS;
      return tile_row8<D>((i & 1) ? On : Qn, 32 * mt + n, 2 * ks + h);
    };
    // Product bundle j: (j even: dV from dO^T, odd: dK from Q^T) of K-step
    // kk, d-tile dt.
    auto atr = [&](int j) {
      const int jj = j >> 1;
      return tile_a_tr<D>((j & 1) ? Qc : Oc, trc, jj / (D / 32), jj % (D / 32));
    };
    f32x16 snext[BQ / 32], dpnext[BQ / 32];
#pragma unroll
    for (int mt = 0; mt < BQ / 32; ++mt) {
      snext[mt] = (f32x16){};
      dpnext[mt] = dp_init(Dn, mt);
    }
    bf16x8 aop[NS], top[NP], pop[BQ / 16], dsop[BQ / 16];
    constexpr int GB = 4 / EPB;  // bundles per 4-row group
    constexpr int LDA = 2;  // groups of L, D in flight ahead of their use
#pragma unroll
    for (int g = 0; g < LDA && g < BQ / 8; ++g) {
      lb[g] = lrow(g);
      if constexpr (DROP) dl[g] = drow(g);
    }
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) aop[i] = arow(i);
    // P/dS element e in three stages: a) the exponent, b) the exponential
    // and dP - D (dropout applied), c) dS = P (dP - D) and the bf16 packs.
    float ea[BQ / 2], eb_p[BQ / 2], eb_d[BQ / 2];
    auto stage_a = [&](int e) {
      const int mt2 = e >> 4, r = e & 15, g = 4 * mt2 + (r >> 2);
      ea[e] = fmaf(scur[mt2][r], s2, -lb[g][r & 3]);
    };
    auto stage_b = [&](int e) {
      const int mt2 = e >> 4, r = e & 15, g = 4 * mt2 + (r >> 2);
      float pv = fast_exp2(ea[e]), dpv = dpcur[mt2][r];
      if constexpr (DROP) {
        const bool kp = dropout_keep(keepw[mt2], r, p.drop.thresh);
        dpv = kp ? dpv * p.drop.inv_keep : 0.f;
        pop[e >> 3][e & 7] = (__bf16)(kp ? pv : 0.f);
      } else {
        pop[e >> 3][e & 7] = (__bf16)pv;
      }
      eb_p[e] = pv;
      if constexpr (DROP)
        eb_d[e] = dpv - dl[g][r & 3];
      else
        eb_d[e] = dpv;  // D - dP from the MFMAs
    };
    auto stage_c = [&](int e) { dsop[e >> 3][e & 7] = (__bf16)(eb_p[e] * eb_d[e]); };
    // The last two bundles' elements (from EPB (NS - 2) on) finish in product
    // bundles 0 and 1; their K-step is first read at product bundle 2 (D/32) kk.
    static_assert(2 * (D / 32) * ((EPB * (NS - 2)) / 8) > 1, "late elements read too early");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + AHEAD < NS) aop[i + AHEAD] = arow(i + AHEAD);
      if (i >= NS - AHEAD) top[i - (NS - AHEAD)] = atr(i - (NS - AHEAD));
      if (i % GB == 0 && i / GB + LDA < BQ / 8) {
        lb[i / GB + LDA] = lrow(i / GB + LDA);
        if constexpr (DROP) dl[i / GB + LDA] = drow(i / GB + LDA);
      }
      const int j = i >> 1, mt = j / KS, ks = j % KS;
      if (i & 1)
        dpnext[mt] = mfma32(aop[i], vop[ks], dpnext[mt]);
      else
        snext[mt] = mfma32(aop[i], kop[ks], snext[mt]);
      // Three elements at different stages, so that their dependent chains
      // overlap instead of stalling this (only) wave of the SIMD.
#pragma unroll
      for (int u = 0; u < EPB; ++u) {
        const int e = EPB * i + u;
        if (e >= 2 * EPB) stage_c(e - 2 * EPB);
        if (e >= EPB) stage_b(e - EPB);
        stage_a(e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j + AHEAD < NP) top[j + AHEAD] = atr(j + AHEAD);
      const int jj = j >> 1, kk = jj / (D / 32), dt = jj % (D / 32);
      if (j & 1)
        dkacc[dt] = mfma32(top[j], dsop[kk], dkacc[dt]);
      else
        dvacc[dt] = mfma32(top[j], pop[kk], dvacc[dt]);
      // The last two bundles' elements finish here, long before the K-step
      // that reads them (the last one, from product bundle 6 (D / 32) on).
      if (j < 2) {
#pragma unroll
        for (int u = 0; u < EPB; ++u) {
          const int e = EPB * (NS - 2 + j) + u;
          stage_c(e);
          if (j == 0) stage_b(e + EPB);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Tile t+2 has landed for every wave; slot c may be refilled next time.
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int mt = 0; mt < BQ / 32; ++mt) {
      scur[mt] = snext[mt];
      dpcur[mt] = dpnext[mt];
    }
  };

  const int U = G * (t_hi - t_lo);  // tiles in the sequence
  for (int u = 0; u < U; u += 3) {
    iteration(sQ0, sO0, sL0, sD0, sQ1, sO1, sD1, sQ2, sO2, sL2, sD2);
    if (u + 1 < U) iteration(sQ1, sO1, sL1, sD1, sQ2, sO2, sD2, sQ0, sO0, sL0, sD0);
    if (u + 2 < U) iteration(sQ2, sO2, sL2, sD2, sQ0, sO0, sD0, sQ1, sO1, sL1, sD1);
  }

  // With the group split, this share's partial sums go to the workspace.
  float* dk_out = p.dk;
  float* dv_out = p.dv;
  if (p.split > 1) {
    const size_t part = (size_t)(gridDim.x / p.n_tiles / p.split) * N * D;
    dk_out = p.dk_part + share * part;
    dv_out = p.dv_part + share * part;
  }
  if (my_k < N) {
    const size_t row = head + (size_t)my_k * D;
    const float vs = DROP ? p.drop.inv_keep : 1.f;
    const float ks_ = DROP ? p.scale : -p.scale;  // (dS negated without dropout)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        *(f32x4*)(dk_out + row + d0) =
            (f32x4){dkacc[dt][4 * g] * ks_, dkacc[dt][4 * g + 1] * ks_,
                    dkacc[dt][4 * g + 2] * ks_, dkacc[dt][4 * g + 3] * ks_};
        if constexpr (DROP)
          *(f32x4*)(dv_out + row + d0) =
              (f32x4){dvacc[dt][4 * g] * vs, dvacc[dt][4 * g + 1] * vs,
                      dvacc[dt][4 * g + 2] * vs, dvacc[dt][4 * g + 3] * vs};
        else
          *(f32x4*)(dv_out + row + d0) = (f32x4){dvacc[dt][4 * g], dvacc[dt][4 * g + 1],
                                                 dvacc[dt][4 * g + 2], dvacc[dt][4 * g + 3]};
      }
  }
}

// --------------------------------------------------- dK, dV (four roles)
// d = 128 without dropout.  The kernel above needs about 340 registers per
// wave at d = 128, so it runs one wave per SIMD, which alternates between
// matrix and vector work.  Here the four products of a key block are split
// over four kinds of wave, and each wave keeps 64 keys of its product, so
// that each operand tile read from LDS feeds two MFMAs (one per 32-key tile;
// with 32 keys per wave the CU's LDS, which takes one wave instruction every
// 4-5 clocks, would be issuing about two instructions per MFMA):
//  * S wave (K^T resident): S = Q K^T of query tile s+1 and, between those
//    MFMAs, P = exp2(s log2(e) S - L log2(e)) of tile s, written (fp32) to
//    an LDS exchange buffer;
//  * dP wave (-V^T resident): D - dP of tile s (the MFMAs start from D) and
//    dS = P (dP - D) of tile s-1 (negated; P from the exchange), written
//    (bf16) to a second exchange buffer;
//  * dV wave: dV^T += dO^T P of tile s-2 (P rounded to bf16);
//  * dK wave: dK^T += Q^T dS of tile s-3.
// Two groups of 64 keys make the workgroup's 128 keys and 8 waves.  The
// waves of a workgroup are placed on the SIMDs round-robin, so waves 0-3 =
// S, dP, S, dP and 4-7 = dK, dV, dK, dV put one wave with vector work (the
// exponentials, or dS) and one with MFMAs (and the rounding of P to bf16)
// on every SIMD, with 32 MFMAs per step each.  Every value is formed as in
// the kernel above, and each accumulator takes its products in the same
// order.
//
// Query tiles of 32 rows (Q, dO, L, D) sit in slot t % 6 of their rings,
// one LDS array per slot (so that the compiler sees that a read of one slot
// does not alias the direct loads into another and inserts no wait for
// them); tile s+3 is fetched at step s and waited for at its end.  Every
// wave reads all the operands of its next step (A tiles, and P or dS from
// the exchange) during the current one, each register taking the next
// tile's operand right after the MFMA that used it, so that no step starts
// by waiting for LDS: the dV and dK waves run two and three tiles behind
// the S wave, which is what lets them read P and dS a step after these
// were written.  P of tile s goes to exchange buffer s % 2, dS of tile s-1
// to buffer (s-1) % 2.  The loop runs U + 3 steps, one barrier each.
template <int V>
using IC = std::integral_constant<int, V>;

// Heads per group of the causal walk of the kernel below (see causal_group):
// two, against four for the other kernels.  Measured on one box (causal
// dK/dV launch, ms): B4 H16 N2048 0.186 with two or four heads, N4096 0.558
// / 0.559, B2 H32 N8192 1.985 / 2.017, B1 H32 N16384 3.71 / 3.86; one head
// per group is slower at N <= 4096 (0.21 and 0.58).
constexpr int kQuadCausalGroup = 2;

template <int D>
__global__ __launch_bounds__(512, 2) void bwd_dkdv_quad_kernel(BwdKParams p) {
  constexpr int BQ = 32;               // query rows per step
  constexpr int NWV = 8;               // waves
  constexpr int BKV = 128;             // keys per workgroup
  constexpr int KS = D / 16;           // K-steps of S and dP
  constexpr int DT = D / 32;           // d-tiles of dK and dV
  constexpr int LDROWS = 64;           // L and D are staged one dword per lane
  constexpr int PF = 2 * 8 * 64 * 4;   // floats of a P buffer: 2 groups x 8 chunks per lane
  constexpr int SH = 2 * 4 * 64 * 8;   // bf16 of a dS buffer: 2 groups x 4 chunks per lane
  static_assert(D == 128, "four-role dK/dV kernel is for d = 128");
  __shared__ __attribute__((aligned(16))) __bf16 sQ0[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ1[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ2[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ3[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ4[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ5[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO0[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO1[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO2[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO3[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO4[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO5[BQ * D];
  __shared__ __attribute__((aligned(16))) float sL0[LDROWS], sL1[LDROWS], sL2[LDROWS], sL3[LDROWS],
      sL4[LDROWS], sL5[LDROWS];
  __shared__ __attribute__((aligned(16))) float sD0[LDROWS], sD1[LDROWS], sD2[LDROWS], sD3[LDROWS],
      sD4[LDROWS], sD5[LDROWS];
  __shared__ __attribute__((aligned(16))) float sP0[PF];
  __shared__ __attribute__((aligned(16))) float sP1[PF];
  __shared__ __attribute__((aligned(16))) __bf16 sS0[SH];
  __shared__ __attribute__((aligned(16))) __bf16 sS1[SH];
  // Slot j (any integer constant, taken mod 6) of each ring; buffer j % 2.
  auto sq = [&](auto J) -> __bf16* {
    constexpr int j = (decltype(J)::value % 6 + 6) % 6;
    if constexpr (j == 0) return sQ0; else if constexpr (j == 1) return sQ1;
    else if constexpr (j == 2) return sQ2; else if constexpr (j == 3) return sQ3;
    else if constexpr (j == 4) return sQ4; else return sQ5;
  };
  auto so = [&](auto J) -> __bf16* {
    constexpr int j = (decltype(J)::value % 6 + 6) % 6;
    if constexpr (j == 0) return sO0; else if constexpr (j == 1) return sO1;
    else if constexpr (j == 2) return sO2; else if constexpr (j == 3) return sO3;
    else if constexpr (j == 4) return sO4; else return sO5;
  };
  auto sl = [&](auto J) -> float* {
    constexpr int j = (decltype(J)::value % 6 + 6) % 6;
    if constexpr (j == 0) return sL0; else if constexpr (j == 1) return sL1;
    else if constexpr (j == 2) return sL2; else if constexpr (j == 3) return sL3;
    else if constexpr (j == 4) return sL4; else return sL5;
  };
  auto sd = [&](auto J) -> float* {
    constexpr int j = (decltype(J)::value % 6 + 6) % 6;
    if constexpr (j == 0) return sD0; else if constexpr (j == 1) return sD1;
    else if constexpr (j == 2) return sD2; else if constexpr (j == 3) return sD3;
    else if constexpr (j == 4) return sD4; else return sD5;
  };
  auto sp = [&](auto J) -> float* {
    if constexpr ((decltype(J)::value % 2 + 2) % 2 == 0) return sP0; else return sP1;
  };
  auto ss = [&](auto J) -> __bf16* {
    if constexpr ((decltype(J)::value % 2 + 2) % 2 == 0) return sS0; else return sS1;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int role = w < 4 ? (w & 1) : 3 - (w & 1);          // 0 S, 1 dP, 2 dV, 3 dK
  const int kg = (w >> 1) & 1;                              // key group
  const int h = lane >> 5, n = lane & 31;
  const TileId id =
      tile_order(blockIdx.x, gridDim.x / p.n_tiles, p.n_tiles, p.causal, kQuadCausalGroup);
  const int bkv = id.bh / p.split;  // key/value head (b * Hkv + hk)
  const int share = id.bh % p.split;
  const int kt = id.rank;
  const int N = p.N, W = p.window;
  const int G = p.H / p.Hkv / p.split;  // query heads this workgroup walks
  const int bh0 = (bkv / p.Hkv) * p.H + (bkv % p.Hkv) * (p.H / p.Hkv) + share * G;
  const int k0 = kt * BKV;
  const int kg0 = k0 + 64 * kg;  // first key of this wave's group; tile t starts at kg0 + 32 t
  const size_t head = (size_t)bkv * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;

  // Queries that can see any key of this block.
  const int k_last = min(k0 + BKV, N) - 1;
  int q_lo = p.causal ? k0 : 0, q_hi = N;
  if (W > 0) {
    q_lo = max(q_lo, k0 - W + 1);
    q_hi = min(q_hi, k_last + W);
  }
  const int t_lo = q_lo / BQ, t_hi = (q_hi + BQ - 1) / BQ;
  const int U = G * (t_hi - t_lo);  // tiles in the sequence (query head, tile)
  const int NSTEP = U + 3;

  const TrCoord trc(lane);
  // This lane's byte offsets inside a tile (row reads of K-step ks;
  // transposing reads of d-tile dt, rows +0 / +8), in an exchange buffer
  // (chunk c of the lane at + 1024 c) and in an L or D row block.  Hidden
  // from the optimizer at every step: otherwise the compiler hoists one
  // address register per slot and read out of the loop.
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
  uint32_t poff = (uint32_t)((kg * 8 * 64 + lane) * 16);
  uint32_t soff = (uint32_t)((kg * 4 * 64 + lane) * 16);
  uint32_t lhoff = (uint32_t)(16 * h);  // L, D rows 4h .. 4h+3 of group 0
  auto rrow = [&](const __bf16* t, int ks) {
    return *(const bf16x8*)((const char*)t + roff[ks]);
  };
  auto rtr = [&](const __bf16* t, int j) {  // A operand of K-step j / DT, d-tile j % DT
    const int kk = j / DT, dt = j % DT;
    const char* b = (const char*)t + 16 * kk * D * 2;
    return cat4(lds_read_tr16(b + toff[2 * dt]), lds_read_tr16(b + toff[2 * dt + 1]));
  };
  auto rvec4 = [&](const float* t, int g) {  // rows 8g + 4h .. +3
    return *(const f32x4*)((const char*)t + lhoff + 32 * g);
  };

  // Fetch cursor (query head lj of the group, tile lt), three tiles ahead
  // of the step, kept by the dK and dV waves (waves 4-7), which fetch every
  // tile: the S wave's own instruction stream is the step's critical path.
  // The buffer resources span the whole query head (rows past N read as
  // zero) and change only with the head; past the last head they are empty,
  // so the tiles fetched after the last one are zeros.  Wave 4 + f moves
  // 1 KB pieces f and f + 4 of the Q and dO tiles (as tile_load_lds), lane L
  // of piece c the global chunk that the swizzle puts at LDS chunk 64 c + L.
  constexpr int NFW = 4;  // fetching waves
  static_assert(BQ * D / 8 == 2 * 64 * NFW, "two 16-byte chunks per lane and tile");
  const bool fetcher = w >= NWV - NFW;
  const int fw = w - (NWV - NFW);
  int lj = 0, lt = t_lo;
  uint32_t chunk_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pc = (fw + NFW * i) * 64 + lane, row = pc / (D / 8);
    const int ch = (pc % (D / 8)) ^ swz<D>(row);
    chunk_off[i] = (uint32_t)(row * D + ch * 8) * 2u;
  }
  __amdgpu_buffer_rsrc_t rq, ro, rl, rd;
  auto set_head = [&]() {
    const bool live = lj < G;
    const int bhq = bh0 + min(lj, G - 1);
    rq = make_rsrc(p.q + (size_t)bhq * N * D, live ? head_bytes : 0u);
    ro = make_rsrc(p.dout + (size_t)bhq * N * D, live ? head_bytes : 0u);
    rl = make_rsrc(p.lse2 + (size_t)bhq * N, live ? (uint32_t)N * 4 : 0u);
    rd = make_rsrc(p.delta + (size_t)bhq * N, live ? (uint32_t)N * 4 : 0u);
  };
  set_head();
  auto load_tile = [&](auto J) {
    if (!fetcher) return;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t voff = chunk_off[i] + (uint32_t)lt * (BQ * D * 2);
      const int c = fw + NFW * i;  // piece of the tile
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (LDS_AS void*)(sq(J) + c * 64 * 8), 16,
                                               (int)voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (LDS_AS void*)(so(J) + c * 64 * 8), 16,
                                               (int)voff, 0, 0, 0);
    }
    if (fw == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (LDS_AS void*)sl(J), 4,
                                               (int)((uint32_t)(lt * BQ + lane) * 4u), 0, 0, 0);
    if (fw == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (LDS_AS void*)sd(J), 4,
                                               (int)((uint32_t)(lt * BQ + lane) * 4u), 0, 0, 0);
    if (++lt == t_hi) {
      lt = t_lo;
      ++lj;
      set_head();
    }
  };
  // Only the offsets that a role uses are hidden (and so kept) in its loop.
  auto hide_offsets = [&]() {
    if (role < 2) {
#pragma unroll
      for (int i = 0; i < KS; ++i) asm volatile("" : "+v"(roff[i]));
      asm volatile("" : "+v"(lhoff));
    } else {
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) asm volatile("" : "+v"(toff[i]));
    }
    if (role != 3) asm volatile("" : "+v"(poff));
    if (role & 1) asm volatile("" : "+v"(soff));
  };
  // Step s (slot j = s % 6) fetches tile s+3.
  auto begin_step = [&](auto J) {
    load_tile(IC<decltype(J)::value + 3>());
    hide_offsets();
  };
  // This step's tile has landed (for every wave after the barrier).
  auto end_step = [&]() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
  };
  // Steps 0 .. NSTEP-1, unrolled by six (slot j = s % 6).
  auto run = [&](auto&& step) {
    int s = 0;
    for (; s + 6 <= NSTEP; s += 6) {
      step(IC<0>(), s);
      step(IC<1>(), s + 1);
      step(IC<2>(), s + 2);
      step(IC<3>(), s + 3);
      step(IC<4>(), s + 4);
      step(IC<5>(), s + 5);
    }
    if (s < NSTEP) step(IC<0>(), s);
    if (s + 1 < NSTEP) step(IC<1>(), s + 1);
    if (s + 2 < NSTEP) step(IC<2>(), s + 2);
    if (s + 3 < NSTEP) step(IC<3>(), s + 3);
    if (s + 4 < NSTEP) step(IC<4>(), s + 4);
  };

  // Prologue: tiles 0 to 2; the slots that the dK and dV waves read before
  // their first tiles arrive (Q slots 4 and 5, dO slot 5) are cleared.
  load_tile(IC<0>());
  load_tile(IC<1>());
  load_tile(IC<2>());
  for (int i = tid; i < BQ * D / 8; i += NWV * 64) {
    ((u32x4*)sQ4)[i] = (u32x4){};
    ((u32x4*)sQ5)[i] = (u32x4){};
    ((u32x4*)sO5)[i] = (u32x4){};
  }

  if (role == 0) {
    // ---- S wave
    bf16x8 bop[2][KS];  // K^T: lane = key, 8 consecutive d per K-step
    {
      const auto r = make_rsrc(p.k + head, head_bytes);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          bop[t][ks] = __builtin_bit_cast(
              bf16x8, buf_load16(r, (uint32_t)((kg0 + 32 * t + n) * D + 16 * ks + 8 * h) * 2u));
    }
    // Queries that see key kg0 + 32 t + n.
    int qmin[2], qmax[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int my_k = kg0 + 32 * t + n;
      qmin[t] = p.causal ? my_k : INT_MIN;
      qmax[t] = INT_MAX;
      if (W > 0) {
        if (!p.causal) qmin[t] = my_k - W + 1;
        qmax[t] = my_k + W - 1;
      }
    }
    const float s2 = p.scale * kLog2e;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    f32x16 cur[2] = {};  // S of the current tile (raw, unmasked)
    bf16x8 aop[KS];      // rows of Q of the next tile
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a0 = rrow(sQ0, ks);
#pragma unroll
      for (int t = 0; t < 2; ++t) cur[t] = mfma32(a0, bop[t][ks], cur[t]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aop[ks] = rrow(sQ1, ks);
    f32x4 lb[4];  // L log2(e) of the rows this lane holds (register 4g + c: row 8g + 4h + c)
#pragma unroll
    for (int g = 0; g < 4; ++g) lb[g] = rvec4(sL0, g);
    int ct = t_lo;
    run([&](auto J, int) {
      begin_step(J);
      const int i0 = ct * BQ;  // first query of tile s
      if (++ct == t_hi) ct = t_lo;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kw0 = kg0 + 32 * t;
        bool need_mask = false;
        if (p.causal) need_mask |= i0 < kw0 + 31;
        if (W > 0) {
          need_mask |= (i0 + BQ - 1) - kw0 >= W;
          if (!p.causal) need_mask |= (kw0 + 31) - i0 >= W;
        }
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = i0 + 8 * (r >> 2) + 4 * h + (r & 3);
            cur[t][r] = (q < qmin[t] || q > qmax[t]) ? -__builtin_inff() : cur[t][r];
          }
        }
      }
      const __bf16* qx = sq(IC<decltype(J)::value + 2>());  // Q of tile s+2
      char* pw = (char*)sp(J);
      f32x16 snext[2] = {};
      float pv[32];
      __builtin_amdgcn_sched_barrier(0);
      // S of tile s+1 (operands read during the step before); four elements
      // of P of tile s per K-step (element e = 16 t + r is register r of
      // tile t; chunk e / 4 is complete after K-step e / 4 and goes out at
      // once); each operand register takes the next tile's row once used.
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          snext[t] = mfma32(aop[ks], bop[t][ks], snext[t]);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 4 * ks + 2 * t + u, te = e >> 4, r = e & 15;
            pv[e] = fast_exp2(fmaf(cur[te][r], s2, -lb[r >> 2][r & 3]));
          }
        }
        aop[ks] = rrow(qx, ks);
        *(f32x4*)(pw + poff + 1024 * ks) =
            (f32x4){pv[4 * ks], pv[4 * ks + 1], pv[4 * ks + 2], pv[4 * ks + 3]};
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) lb[g] = rvec4(sl(IC<decltype(J)::value + 1>()), g);
      cur[0] = snext[0];
      cur[1] = snext[1];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): P of tile s is in LDS
      end_step();
    });
  } else if (role == 1) {
    // ---- dP wave
    bf16x8 bop[2][KS];  // -V^T
    {
      const auto r = make_rsrc(p.v + head, head_bytes);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          bop[t][ks] = __builtin_bit_cast(
              bf16x8,
              buf_load16(r, (uint32_t)((kg0 + 32 * t + n) * D + 16 * ks + 8 * h) * 2u) ^
                  0x80008000u);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    f32x16 cur[2] = {};  // D - dP of the tile before the current one
    bf16x8 aop[KS];      // rows of dO of the current tile
    f32x4 dv[4];         // D of the rows this lane holds
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aop[ks] = rrow(sO0, ks);
#pragma unroll
    for (int g = 0; g < 4; ++g) dv[g] = rvec4(sD0, g);
    run([&](auto J, int) {
      begin_step(J);
      f32x16 dpn[2];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int c = 0; c < 4; ++c) dpn[0][4 * g + c] = dv[g][c];
      dpn[1] = dpn[0];
      const char* pr = (const char*)sp(IC<decltype(J)::value + 1>());  // P of tile s-1
      char* sw = (char*)ss(IC<decltype(J)::value + 1>());              // dS of tile s-1
      const __bf16* ox = so(IC<decltype(J)::value + 1>());             // dO of tile s+1
      f32x4 pp[8];
      bf16x8 dsop[2][2];
      __builtin_amdgcn_sched_barrier(0);
      // D - dP of tile s, and dS of tile s-1 from K-step 2 on (elements
      // EB[ks] .. EB[ks+1]-1 in K-step ks; element e = 16 t + r is register
      // r of key tile t), so that the first MFMAs do not wait for P, which
      // is read from K-step 0 on; chunk e / 8 of dS goes out once complete;
      // each operand register takes the next tile's row once used.
      constexpr int EB[KS + 1] = {0, 0, 0, 4, 10, 16, 22, 28, 32};
      constexpr int PK[8] = {0, 0, 1, 2, 3, 3, 4, 5};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // P chunk c is read in K-step PK[c], at least one K-step before use.
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (PK[c] == ks) pp[c] = *(const f32x4*)(pr + poff + 1024 * c);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          dpn[t] = mfma32(aop[ks], bop[t][ks], dpn[t]);
          const int half = (EB[ks + 1] - EB[ks]) / 2;
          const int e0 = EB[ks] + t * half, e1 = t ? EB[ks + 1] : EB[ks] + half;
#pragma unroll
          for (int u = 0; u < 4; ++u) {  // constant trip count: fully unrolled
            const int e = e0 + u;
            if (e < e1) {
              const int te = e >> 4, r = e & 15;
              dsop[te][r >> 3][r & 7] = (__bf16)(pp[e >> 2][e & 3] * cur[te][r]);
            }
          }
        }
        aop[ks] = rrow(ox, ks);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (8 * c + 8 > EB[ks] && 8 * c + 8 <= EB[ks + 1])
            *(bf16x8*)(sw + soff + 1024 * c) = dsop[c >> 1][c & 1];
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) dv[g] = rvec4(sd(IC<decltype(J)::value + 1>()), g);
      cur[0] = dpn[0];
      cur[1] = dpn[1];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): dS of tile s-1 is in LDS
      end_step();
    });
  } else {
    // ---- dV wave (role 2: tile s-2 at step s) and dK wave (role 3: tile s-3)
    const bool vwave = role == 2;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    f32x16 acc[2][DT];  // dV^T, or -dK^T / s, of key tiles 0 and 1
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[t][dt] = (f32x16){};
    bf16x8 top[2 * DT];  // A operands (K-step j / DT, d-tile j % DT), read the step before
    bf16x8 bo[2][2];     // B operands (P or dS, bf16) of key tile t, K-step kk
#pragma unroll
    for (int j = 0; j < 2 * DT; ++j) top[j] = (bf16x8){};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) bo[t][kk] = (bf16x8){};
    // This step's products, each A operand register taking the next tile's
    // operand once used.  The MFMAs run at every step; outside a wave's
    // tiles its A and B operands are zero (the slots read before the first
    // tile arrives were cleared, the tiles after the last one are fetched
    // as zeros), so they add exactly nothing whatever the inputs hold.
    auto product = [&](const __bf16* ax) {
#pragma unroll
      for (int j = 0; j < 2 * DT; ++j) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][j % DT] = mfma32(top[j], bo[t][j / DT], acc[t][j % DT]);
        top[j] = rtr(ax, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (vwave) {
      // Step s: dV += dO_{s-2}^T P_{s-2}; reads dO of tile s-1 (slot s+5)
      // and P of tile s-1 (buffer s+1).
      run([&](auto J, int s) {
        begin_step(J);
        __builtin_amdgcn_sched_barrier(0);
        product(so(IC<decltype(J)::value + 5>()));
        const char* pr = (const char*)sp(IC<decltype(J)::value + 1>());
        const bool next = s + 1 >= 2 && s + 1 <= U + 1;  // dV of tile s-1 at step s+1
        f32x4 pp[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) pp[c] = *(const f32x4*)(pr + poff + 1024 * c);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            bf16x8 b;
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = (__bf16)pp[4 * t + 2 * kk + (j >> 2)][j & 3];
            bo[t][kk] = next ? b : (bf16x8){};
          }
        end_step();
      });
    } else {
      // Step s: dK += Q_{s-3}^T dS_{s-3}; reads Q of tile s-2 (slot s+4)
      // and dS of tile s-2 (buffer s).
      run([&](auto J, int s) {
        begin_step(J);
        __builtin_amdgcn_sched_barrier(0);
        product(sq(IC<decltype(J)::value + 4>()));
        const char* sr = (const char*)ss(J);
        const bool next = s + 1 >= 3;  // dK of tile s-2 at step s+1
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 b = *(const bf16x8*)(sr + soff + 1024 * (2 * t + kk));
            bo[t][kk] = next ? b : (bf16x8){};
          }
        end_step();
      });
    }
    __builtin_amdgcn_s_waitcnt(0);  // no load may land after the workgroup ends
    // With the group split, this share's partial sums go to the workspace.
    float* out = vwave ? p.dv : p.dk;
    if (p.split > 1) {
      const size_t part = (size_t)(gridDim.x / p.n_tiles / p.split) * N * D;
      out = (vwave ? p.dv_part : p.dk_part) + share * part;
    }
    const float sc = vwave ? 1.f : -p.scale;  // (dS negated)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int my_k = kg0 + 32 * t + n;
      if (my_k < N) {
        const size_t row = head + (size_t)my_k * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(f32x4*)(out + row + 32 * dt + 8 * g + 4 * h) =
                (f32x4){acc[t][dt][4 * g] * sc, acc[t][dt][4 * g + 1] * sc,
                        acc[t][dt][4 * g + 2] * sc, acc[t][dt][4 * g + 3] * sc};
      }
    }
    return;
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land after the workgroup ends
}

// --------------------------------------------------- dK, dV ping-pong (d = 64)
// d = 64 without dropout or causal mask: workgroups of 8 waves (256 keys, 32 per wave, K^T
// and -V^T resident), split into two groups one half-step apart as in the
// ping-pong forward: M(u) issues the S and D - dP MFMAs of query tile u+1
// and dV^T += dO_u^T P_u, dK^T += Q_u^T dS_u (16 MFMAs, the four kinds
// alternating), V(u) masks and forms P and dS of tile u+1; a barrier ends
// every half-step.  Query tiles of 32 rows (Q by waves 0-3, dO by waves 4-7,
// L and D by waves 0 and 1) sit in slot j % 4 of their rings; tile u+3 is
// fetched at half-step 2u, every half-step ends by waiting for the fetches of
// two half-steps before, and a wave reads the first operands of its next M
// in its V.  The walk over the group's query heads and the split into
// shares are those of bwd_dkdv_kernel; values and accumulation order too.
template <int D, int NG>
__global__ __launch_bounds__(2 * NG * 64, 2) void bwd_dkdv_pp_kernel(BwdKParams p) {
  constexpr int BQ = 32;
  constexpr int NWV = 2 * NG;
  constexpr int BKV = 32 * NWV;
  constexpr int KS = D / 16, DT = D / 32;
  static_assert(KS == (BQ / 16) * DT, "S, dP, dV and dK products alternate one to one");
  constexpr int NM = 4 * KS;
  constexpr int AHEAD = 3;
  constexpr int LDROWS = 64;
  __shared__ __attribute__((aligned(16))) __bf16 sQ0[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ1[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ2[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sQ3[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO0[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO1[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO2[BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sO3[BQ * D];
  __shared__ __attribute__((aligned(16))) float sL0[LDROWS], sL1[LDROWS], sL2[LDROWS], sL3[LDROWS];
  __shared__ __attribute__((aligned(16))) float sD0[LDROWS], sD1[LDROWS], sD2[LDROWS], sD3[LDROWS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const bool lead = w < NG;
  const int h = lane >> 5, n = lane & 31;
  const TileId id =
      tile_order(blockIdx.x, gridDim.x / p.n_tiles, p.n_tiles, p.causal, causal_group<D>());
  const int bkv = id.bh / p.split;
  const int share = id.bh % p.split;
  const int kt = id.rank;
  const int N = p.N, W = p.window;
  const int G = p.H / p.Hkv / p.split;
  const int bh0 = (bkv / p.Hkv) * p.H + (bkv % p.Hkv) * (p.H / p.Hkv) + share * G;
  const int k0 = kt * BKV;
  const int kw0 = k0 + 32 * w;
  const int my_k = kw0 + n;
  const size_t head = (size_t)bkv * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;

  // K^T and -V^T as B operands (lane = key); the dP MFMAs start from D_i
  // and take -V, leaving D_i - dP_ij, and dS comes out negated.
  bf16x8 kop[KS], vop[KS];
  {
    const auto rk = make_rsrc(p.k + head, head_bytes);
    const auto rv = make_rsrc(p.v + head, head_bytes);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off = (uint32_t)(my_k * D + 16 * ks + 8 * h) * 2u;
      kop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
      vop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rv, off) ^ 0x80008000u);
    }
  }
  f32x16 dkacc[DT], dvacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dkacc[dt] = dvacc[dt] = (f32x16){};

  const int k_last = min(k0 + BKV, N) - 1;
  int q_lo = p.causal ? k0 : 0, q_hi = N;
  int qmin = p.causal ? my_k : INT_MIN, qmax = INT_MAX;
  if (W > 0) {
    q_lo = max(q_lo, k0 - W + 1);
    q_hi = min(q_hi, k_last + W);
    if (!p.causal) qmin = my_k - W + 1;
    qmax = my_k + W - 1;
  }
  const int t_lo = q_lo / BQ, t_hi = (q_hi + BQ - 1) / BQ;
  const int T = G * (t_hi - t_lo);  // tiles in the walk (query head, tile)

  const float s2 = p.scale * kLog2e;
  const TrCoord trc(lane);
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
  uint32_t lhoff = (uint32_t)(16 * h);
  auto hide = [&]() {
#pragma unroll
    for (int i = 0; i < KS; ++i) asm volatile("" : "+v"(roff[i]));
#pragma unroll
    for (int i = 0; i < 2 * DT; ++i) asm volatile("" : "+v"(toff[i]));
    asm volatile("" : "+v"(lhoff));
  };
  auto rrow = [&](const __bf16* t, int ks) {
    return *(const bf16x8*)((const char*)t + roff[ks]);
  };
  auto rtr = [&](const __bf16* t, int j) {  // K-step j / DT, d-tile j % DT
    const char* b = (const char*)t + 16 * (j / DT) * D * 2;
    return cat4(lds_read_tr16(b + toff[2 * (j % DT)]), lds_read_tr16(b + toff[2 * (j % DT) + 1]));
  };
  auto rvec4 = [&](const float* t, int g) {  // rows 8g + 4h .. +3
    return *(const f32x4*)((const char*)t + lhoff + 32 * g);
  };

  // Load cursor over the walk; past the last head it keeps reading the last
  // head's rows (in bounds, never used).
  int lj = 0, lt = t_lo, ct = t_lo;
  auto load_tile = [&](__bf16* Qf, __bf16* Of, float* Lf, float* Df) {
    const int bhq = bh0 + min(lj, G - 1);
    const size_t qhead = (size_t)bhq * N * D;
    if (lead)
      tile_load_lds<D, BQ, NG>(p.q + qhead, head_bytes, lt * BQ, Qf, w, lane);
    else
      tile_load_lds<D, BQ, NG>(p.dout + qhead, head_bytes, lt * BQ, Of, w - NG, lane);
    if (w == 0)
      vec_load_lds<LDROWS>(make_rsrc(p.lse2 + (size_t)bhq * N, (uint32_t)N * 4), lt * BQ,
                           Lf, lane);
    if (w == 1)
      vec_load_lds<LDROWS>(make_rsrc(p.delta + (size_t)bhq * N, (uint32_t)N * 4), lt * BQ,
                           Df, lane);
    if (++lt == t_hi) {
      lt = t_lo;
      ++lj;
    }
  };

  f32x16 snx, dpnx;  // S and D - dP of the tile whose P and dS come next
  bf16x8 pop[2], dsop[2];
  // Mask (query tile starting at i0), P = exp2(S s2 - L log2 e) and dS (negated).
  auto ds_step = [&](int i0, const float* Lc) {
    bool need_mask = false;
    if (p.causal) need_mask |= i0 < kw0 + 31;
    if (W > 0) {
      need_mask |= (i0 + BQ - 1) - kw0 >= W;
      if (!p.causal) need_mask |= (kw0 + 31) - i0 >= W;
    }
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = i0 + 8 * (r >> 2) + 4 * h + (r & 3);
        snx[r] = (q < qmin || q > qmax) ? -__builtin_inff() : snx[r];
      }
    }
    f32x4 lb[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) lb[g] = rvec4(Lc, g);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = fast_exp2(fmaf(snx[e], s2, -lb[e >> 2][e & 3]));
      pop[e >> 3][e & 7] = (__bf16)pv;
      dsop[e >> 3][e & 7] = (__bf16)(pv * dpnx[e]);
    }
  };
  auto dp_init = [&](const float* Ds) {
    f32x16 c;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = rvec4(Ds, g);
#pragma unroll
      for (int i = 0; i < 4; ++i) c[4 * g + i] = v[i];
    }
    return c;
  };

  // Prologue: tiles 0, 1, 2; S, D - dP, P and dS of tile 0.
  load_tile(sQ0, sO0, sL0, sD0);
  load_tile(sQ1, sO1, sL1, sD1);
  load_tile(sQ2, sO2, sL2, sD2);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  hide();
  snx = (f32x16){};
  dpnx = dp_init(sD0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    snx = mfma32(tile_row8<D>(sQ0, n, 2 * ks + h), kop[ks], snx);
    dpnx = mfma32(tile_row8<D>(sO0, n, 2 * ks + h), vop[ks], dpnx);
  }
  ds_step(ct * BQ, sL0);
  if (++ct == t_hi) ct = t_lo;

  auto end_half = [&]() {
    if (w < 2)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(1));
    __builtin_amdgcn_s_barrier();
  };
  auto fetch = [&](__bf16* Qf, __bf16* Of, float* Lf, float* Df) { load_tile(Qf, Of, Lf, Df); };
  // M(u) operand i: by i % 4 a Q row (S of tile u+1), a dO row (dP of tile
  // u+1), a transposed dO_u pair (dV) or a transposed Q_u pair (dK).
  bf16x8 opd[NM];
  auto issue = [&](int i, const __bf16* Qc, const __bf16* Oc, const __bf16* Qn,
                   const __bf16* On) {
    const int j = i / 4;
    if (i % 4 == 0) opd[i] = rrow(Qn, j);
    else if (i % 4 == 1) opd[i] = rrow(On, j);
    else if (i % 4 == 2) opd[i] = rtr(Oc, j);
    else opd[i] = rtr(Qc, j);
  };
  auto prefetch = [&](const __bf16* Qc, const __bf16* Oc, const __bf16* Qn, const __bf16* On) {
    hide();
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) issue(i, Qc, Oc, Qn, On);
  };
  auto mstep = [&](const __bf16* Qc, const __bf16* Oc, const __bf16* Qn, const __bf16* On,
                   const float* Dn) {
    hide();
    f32x16 s = (f32x16){}, dp = dp_init(Dn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + AHEAD < NM) issue(i + AHEAD, Qc, Oc, Qn, On);
      const int j = i / 4;
      if (i % 4 == 0) s = mfma32(opd[i], kop[j], s);
      else if (i % 4 == 1) dp = mfma32(opd[i], vop[j], dp);
      else if (i % 4 == 2) dvacc[j % DT] = mfma32(opd[i], pop[j / DT], dvacc[j % DT]);
      else dkacc[j % DT] = mfma32(opd[i], dsop[j / DT], dkacc[j % DT]);
      __builtin_amdgcn_sched_barrier(0);
    }
    snx = s;
    dpnx = dp;
  };
  auto vstep = [&](int u, const float* Ln) {
    if (u >= 0 && u + 1 < T) {
      hide();
      ds_step(ct * BQ, Ln);
      if (++ct == t_hi) ct = t_lo;
    }
  };

  // Half-steps 0 .. 2T: the lead group runs M(u) at 2u and V(u) at 2u+1,
  // the other V(u-1) at 2u and M(u) at 2u+1; both end with one more.
  int u = 0;
  if (lead) {
    prefetch(sQ0, sO0, sQ1, sO1);
    for (; u + 4 <= T; u += 4) {
      fetch(sQ3, sO3, sL3, sD3);
      mstep(sQ0, sO0, sQ1, sO1, sD1);
      end_half();
      prefetch(sQ1, sO1, sQ2, sO2);
      vstep(u, sL1);
      end_half();
      fetch(sQ0, sO0, sL0, sD0);
      mstep(sQ1, sO1, sQ2, sO2, sD2);
      end_half();
      prefetch(sQ2, sO2, sQ3, sO3);
      vstep(u + 1, sL2);
      end_half();
      fetch(sQ1, sO1, sL1, sD1);
      mstep(sQ2, sO2, sQ3, sO3, sD3);
      end_half();
      prefetch(sQ3, sO3, sQ0, sO0);
      vstep(u + 2, sL3);
      end_half();
      fetch(sQ2, sO2, sL2, sD2);
      mstep(sQ3, sO3, sQ0, sO0, sD0);
      end_half();
      prefetch(sQ0, sO0, sQ1, sO1);
      vstep(u + 3, sL0);
      end_half();
    }
    if (u < T) {
      fetch(sQ3, sO3, sL3, sD3);
      mstep(sQ0, sO0, sQ1, sO1, sD1);
      end_half();
      prefetch(sQ1, sO1, sQ2, sO2);
      vstep(u, sL1);
      end_half();
    }
    if (u + 1 < T) {
      fetch(sQ0, sO0, sL0, sD0);
      mstep(sQ1, sO1, sQ2, sO2, sD2);
      end_half();
      prefetch(sQ2, sO2, sQ3, sO3);
      vstep(u + 1, sL2);
      end_half();
    }
    if (u + 2 < T) {
      fetch(sQ1, sO1, sL1, sD1);
      mstep(sQ2, sO2, sQ3, sO3, sD3);
      end_half();
      prefetch(sQ3, sO3, sQ0, sO0);
      vstep(u + 2, sL3);
      end_half();
    }
    end_half();
  } else {
    for (; u + 4 <= T; u += 4) {
      fetch(sQ3, sO3, sL3, sD3);
      prefetch(sQ0, sO0, sQ1, sO1);
      vstep(u - 1, sL0);
      end_half();
      mstep(sQ0, sO0, sQ1, sO1, sD1);
      end_half();
      fetch(sQ0, sO0, sL0, sD0);
      prefetch(sQ1, sO1, sQ2, sO2);
      vstep(u, sL1);
      end_half();
      mstep(sQ1, sO1, sQ2, sO2, sD2);
      end_half();
      fetch(sQ1, sO1, sL1, sD1);
      prefetch(sQ2, sO2, sQ3, sO3);
      vstep(u + 1, sL2);
      end_half();
      mstep(sQ2, sO2, sQ3, sO3, sD3);
      end_half();
      fetch(sQ2, sO2, sL2, sD2);
      prefetch(sQ3, sO3, sQ0, sO0);
      vstep(u + 2, sL3);
      end_half();
      mstep(sQ3, sO3, sQ0, sO0, sD0);
      end_half();
    }
    if (u < T) {
      fetch(sQ3, sO3, sL3, sD3);
      prefetch(sQ0, sO0, sQ1, sO1);
      vstep(u - 1, sL0);
      end_half();
      mstep(sQ0, sO0, sQ1, sO1, sD1);
      end_half();
    }
    if (u + 1 < T) {
      fetch(sQ0, sO0, sL0, sD0);
      prefetch(sQ1, sO1, sQ2, sO2);
      vstep(u, sL1);
      end_half();
      mstep(sQ1, sO1, sQ2, sO2, sD2);
      end_half();
    }
    if (u + 2 < T) {
      fetch(sQ1, sO1, sL1, sD1);
      prefetch(sQ2, sO2, sQ3, sO3);
      vstep(u + 1, sL2);
      end_half();
      mstep(sQ2, sO2, sQ3, sO3, sD3);
      end_half();
    }
    end_half();
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land after the workgroup ends

  float* dk_out = p.dk;
  float* dv_out = p.dv;
  if (p.split > 1) {
    const size_t part = (size_t)(gridDim.x / p.n_tiles / p.split) * N * D;
    dk_out = p.dk_part + share * part;
    dv_out = p.dv_part + share * part;
  }
  if (my_k < N) {
    const size_t row = head + (size_t)my_k * D;
    const float ks_ = -p.scale;  // (dS negated)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        *(f32x4*)(dk_out + row + d0) =
            (f32x4){dkacc[dt][4 * g] * ks_, dkacc[dt][4 * g + 1] * ks_,
                    dkacc[dt][4 * g + 2] * ks_, dkacc[dt][4 * g + 3] * ks_};
        *(f32x4*)(dv_out + row + d0) = (f32x4){dvacc[dt][4 * g], dvacc[dt][4 * g + 1],
                                               dvacc[dt][4 * g + 2], dvacc[dt][4 * g + 3]};
      }
  }
}

// out = sum over `split` partial arrays of n4 float4 each (stride n4 apart),
// in share order, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void bwd_share_sum_kernel(const f32x4* part, f32x4* out,
                                                            size_t n4, int split) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * 256) {
    f32x4 acc = part[i];
    for (int s = 1; s < split; ++s) acc += part[s * n4 + i];
    out[i] = acc;
  }
}

// ---------------------------------------------------------------- dQ
// One workgroup per block of 32*NW queries (one query per lane on the MFMA N
// side); K/V tiles of BC keys stream through three LDS slots fetched one
// tile ahead.  Iteration t computes S^T and dP^T of tile t+1 on the matrix
// cores while the VALU forms P and dS^T of tile t, then dQ^T += K_t^T dS_t^T.
// DROP: dS = P (Z dP / keep - D) with the forward's keep bytes.  (Two waves
// per SIMD even though the keep bytes then spill a few registers: measured
// faster than one wave per SIMD without spills.)
template <int D, int NW, int BC, bool DROP>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(BwdKParams p) {
  constexpr int BR = 32 * NW;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) __bf16 sK0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sK1[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sK2[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV1[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV2[BC * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int h = lane >> 5, n = lane & 31;
  const TileId id =
      tile_order(blockIdx.x, gridDim.x / p.n_tiles, p.n_tiles, p.causal, causal_group<D>());
  const int bh = id.bh;
  const int qt = p.causal ? p.n_tiles - 1 - id.rank : id.rank;  // longest first
  const int N = p.N, W = p.window;
  const int q0 = qt * BR;
  const int wq0 = q0 + 32 * w;
  const int my_q = wq0 + n;
  const size_t head = (size_t)bh * N * D;
  const size_t kv_off = (size_t)kv_head(bh, p.H, p.Hkv) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc(p.q + head, head_bytes);
  const __bf16* kh = p.k + kv_off;
  const __bf16* vh = p.v + kv_off;
  const auto rdo = make_rsrc(p.dout + head, head_bytes);
  const auto ro = make_rsrc(p.o + head, head_bytes);

  // Q^T and dO^T as B operands (lane = query): this lane holds d = 16ks +
  // 8h .. +7 of its query for every K-step ks, and the same slice of O_i
  // for its half of D_i = sum_k dO_ik O_ik.
  bf16x8 qop[KS], doop[KS];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)(my_q * D + 16 * ks + 8 * h) * 2u;
    qop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    doop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
    const bf16x8 ov = __builtin_bit_cast(bf16x8, buf_load16(ro, off));
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = fmaf((float)doop[ks][e], (float)ov[e], dpart);
  }
  const bool q_ok = my_q < N;
  const float Lb = q_ok ? p.lse[(size_t)bh * N + my_q] * kLog2e : 0.f;
  const float Dl = halves_sum(dpart);
  // Without dropout the dP^T MFMAs start from D_i and take -dO, so that they
  // leave D_i - dP_ij (as in the dK/dV pass); dS comes out negated and the
  // dQ epilogue multiplies by -s.
  if constexpr (!DROP) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      doop[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, doop[ks]) ^ 0x80008000u);
  }
  const f32x16 dp0 = DROP ? (f32x16){} : (f32x16){Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl,
                                                  Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl};
  // Leave D_i and L_i log2(e) for the dK/dV pass.
  if (q_ok && h == 0) {
    p.delta[(size_t)bh * N + my_q] = Dl;
    p.lse2[(size_t)bh * N + my_q] = Lb;
  }

  const int q_last = min(q0 + BR, N) - 1;
  int kv_lo = 0, kv_hi = N;
  if (p.causal) kv_hi = min(kv_hi, q_last + 1);
  if (W > 0) {
    kv_lo = max(0, q0 - W + 1);
    if (!p.causal) kv_hi = min(kv_hi, q_last + W);
  }
  const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;
  int hi_key = N - 1, lo_key = 0;
  if (p.causal) hi_key = min(hi_key, my_q);
  if (W > 0) {
    lo_key = my_q - W + 1;
    if (!p.causal) hi_key = min(hi_key, my_q + W - 1);
  }

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dqacc[dt] = (f32x16){};
  const float s2 = p.scale * kLog2e;
  const TrCoord trc(lane);

  auto sdp = [&](const __bf16* Ks, const __bf16* Vs, f32x16* sacc, f32x16* dpacc) {
#pragma unroll
    for (int mt = 0; mt < BC / 32; ++mt) {
      sacc[mt] = (f32x16){};
      dpacc[mt] = dp0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sacc[mt] = mfma32(tile_row8<D>(Ks, 32 * mt + n, 2 * ks + h), qop[ks], sacc[mt]);
        dpacc[mt] = mfma32(tile_row8<D>(Vs, 32 * mt + n, 2 * ks + h), doop[ks], dpacc[mt]);
      }
    }
  };

  tile_load_lds<D, BC, NW>(kh, head_bytes, t_lo * BC, sK0, w, lane);
  tile_load_lds<D, BC, NW>(vh, head_bytes, t_lo * BC, sV0, w, lane);
  tile_load_lds<D, BC, NW>(kh, head_bytes, (t_lo + 1) * BC, sK1, w, lane);
  tile_load_lds<D, BC, NW>(vh, head_bytes, (t_lo + 1) * BC, sV1, w, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 scur[BC / 32], dpcur[BC / 32];
  sdp(sK0, sV0, scur, dpcur);

  // Iteration for key tile t: P, dS^T of tile t and dQ^T += K_t^T dS_t^T
  // (K_t in slot c), S^T, dP^T of tile t+1 (slot n); tile t+2 -> slot f.
  auto iteration = [&](int t, const __bf16* Kc, const __bf16* Kn, const __bf16* Vn,
                       __bf16* Kf, __bf16* Vf) {
    tile_load_lds<D, BC, NW>(kh, head_bytes, (t + 2) * BC, Kf, w, lane);
    tile_load_lds<D, BC, NW>(vh, head_bytes, (t + 2) * BC, Vf, w, lane);
    const int kv0 = t * BC;
    bool need_mask = (kv0 + BC > N) || (wq0 + 32 > N);
    if (p.causal) need_mask |= kv0 + BC - 1 > wq0;
    if (W > 0) {
      need_mask |= wq0 + 31 - kv0 >= W;
      if (!p.causal) need_mask |= kv0 + BC - 1 - wq0 >= W;
    }
    if (need_mask) {
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
          scur[mt][r] = (key > hi_key || key < lo_key || !q_ok) ? -__builtin_inff()
                                                                  : scur[mt][r];
        }
    }
    u32x4 keepw[BC / 32];
    if constexpr (DROP) {
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt)
        keepw[mt] = dropout_bytes<false>(p.drop, bh, wq0, kv0 + 32 * mt, lane);
    }
    constexpr int NS = 2 * (BC / 32) * KS;
    constexpr int NP = (BC / 16) * (D / 32);
    constexpr int EPB = (BC / 2) / NS;
    constexpr int AHEAD = 2;
    static_assert(EPB >= 1 && (BC / 2) % NS == 0, "bundle split");
    auto arow = [&](int i) {
      const int j = i >> 1, mt = j / KS, ks = j % KS;
      return tile_row8<D>((i & 1) ? Vn : Kn, 32 * mt + n, 2 * ks + h);
    };
    auto atr = [&](int j) { return tile_a_tr<D>(Kc, trc, j / (D / 32), j % (D / 32)); };
    f32x16 snext[BC / 32], dpnext[BC / 32];
#pragma unroll
    for (int mt = 0; mt < BC / 32; ++mt) {
      snext[mt] = (f32x16){};
      dpnext[mt] = dp0;
    }
    bf16x8 aop[NS], top[NP], dsop[BC / 16];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) aop[i] = arow(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + AHEAD < NS) aop[i + AHEAD] = arow(i + AHEAD);
      if (i >= NS - AHEAD) top[i - (NS - AHEAD)] = atr(i - (NS - AHEAD));
      const int j = i >> 1, mt = j / KS, ks = j % KS;
      if (i & 1)
        dpnext[mt] = mfma32(aop[i], doop[ks], dpnext[mt]);
      else
        snext[mt] = mfma32(aop[i], qop[ks], snext[mt]);
#pragma unroll
      for (int u = 0; u < EPB; ++u) {
        const int e = EPB * i + u, mt2 = e >> 4, r = e & 15;
        const float pv = fast_exp2(fmaf(scur[mt2][r], s2, -Lb));
        float dpv = dpcur[mt2][r];
        if constexpr (DROP)
          dpv = dropout_keep(keepw[mt2], r, p.drop.thresh) ? dpv * p.drop.inv_keep : 0.f;
        dsop[e >> 3][e & 7] = (__bf16)(pv * (DROP ? dpv - Dl : dpv));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j + AHEAD < NP) top[j + AHEAD] = atr(j + AHEAD);
      dqacc[j % (D / 32)] = mfma32(top[j], dsop[j / (D / 32)], dqacc[j % (D / 32)]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int mt = 0; mt < BC / 32; ++mt) {
      scur[mt] = snext[mt];
      dpcur[mt] = dpnext[mt];
    }
  };

  for (int t = t_lo; t < t_hi; t += 3) {
    iteration(t, sK0, sK1, sV1, sK2, sV2);
    if (t + 1 < t_hi) iteration(t + 1, sK1, sK2, sV2, sK0, sV0);
    if (t + 2 < t_hi) iteration(t + 2, sK2, sK0, sV0, sK1, sV1);
  }

  if (q_ok) {
    const size_t row = head + (size_t)my_q * D;
    const float qs = DROP ? p.scale : -p.scale;  // (dS negated without dropout)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        *(f32x4*)(p.dq + row + d0) =
            (f32x4){dqacc[dt][4 * g] * qs, dqacc[dt][4 * g + 1] * qs,
                    dqacc[dt][4 * g + 2] * qs, dqacc[dt][4 * g + 3] * qs};
      }
  }
}

// ------------------------------------------------------------ dQ ping-pong
// d = 128 without dropout: the dQ pass in workgroups of 8 waves (256
// queries) split into two groups one half-step apart, as the forward's
// ping-pong kernel: M(u) issues the S^T and D - dP^T MFMAs of key tile u+1
// and dQ^T += K_u^T dS_u^T (24 MFMAs alternating), V(u) masks and forms P and
// dS^T of tile u+1; a barrier ends every half-step.  K_j and V_j sit in slot
// j % 4 of their rings; at every even half-step 2u the waves fetch K_{u+3}
// and V_{u+3}, every half-step ends by waiting for the fetches of two
// half-steps before, and a wave reads the first operands of its next M in
// its V.  Under the causal mask the first group stops computing after the
// last tile its 128 queries see and then only fetches and joins the
// barriers.  Values and accumulation order are those of bwd_dq_kernel.
template <int D, int NG>
__global__ __launch_bounds__(2 * NG * 64, 2) void bwd_dq_pp_kernel(BwdKParams p) {
  constexpr int BC = 32;
  constexpr int NWV = 2 * NG;
  constexpr int BR = 32 * NWV;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int NM = 3 * KS;  // MFMAs of one M: S, dP and dQ alternating
  constexpr int AHEAD = 3;
  __shared__ __attribute__((aligned(16))) __bf16 sK0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sK1[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sK2[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sK3[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV1[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV2[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV3[BC * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const bool lead = w < NG;
  const int h = lane >> 5, n = lane & 31;
  const TileId id =
      tile_order(blockIdx.x, gridDim.x / p.n_tiles, p.n_tiles, p.causal, causal_group<D>());
  const int bh = id.bh;
  const int qt = p.causal ? p.n_tiles - 1 - id.rank : id.rank;  // longest first
  const int N = p.N, W = p.window;
  const int q0 = qt * BR;
  const int wq0 = q0 + 32 * w;
  const int my_q = wq0 + n;
  const size_t head = (size_t)bh * N * D;
  const size_t kv_off = (size_t)kv_head(bh, p.H, p.Hkv) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc(p.q + head, head_bytes);
  const __bf16* kh = p.k + kv_off;
  const __bf16* vh = p.v + kv_off;
  const auto rdo = make_rsrc(p.dout + head, head_bytes);
  const auto ro = make_rsrc(p.o + head, head_bytes);

  // Q^T and -dO^T as B operands (lane = query), D_i = sum_k dO_ik O_ik.
  bf16x8 qop[KS], doop[KS];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)(my_q * D + 16 * ks + 8 * h) * 2u;
    qop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    doop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
    const bf16x8 ov = __builtin_bit_cast(bf16x8, buf_load16(ro, off));
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = fmaf((float)doop[ks][e], (float)ov[e], dpart);
  }
  const bool q_ok = my_q < N;
  const float Lb = q_ok ? p.lse[(size_t)bh * N + my_q] * kLog2e : 0.f;
  const float Dl = halves_sum(dpart);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    doop[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, doop[ks]) ^ 0x80008000u);
  const f32x16 dp0 = (f32x16){Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl, Dl};
  if (q_ok && h == 0) {
    p.delta[(size_t)bh * N + my_q] = Dl;
    p.lse2[(size_t)bh * N + my_q] = Lb;
  }

  const int q_last = min(q0 + BR, N) - 1;
  int kv_lo = 0, kv_hi = N;
  if (p.causal) kv_hi = min(kv_hi, q_last + 1);
  if (W > 0) {
    kv_lo = max(0, q0 - W + 1);
    if (!p.causal) kv_hi = min(kv_hi, q_last + W);
  }
  const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;
  const int T = t_hi - t_lo;
  int hi_key = N - 1, lo_key = 0;
  if (p.causal) hi_key = min(hi_key, my_q);
  if (W > 0) {
    lo_key = my_q - W + 1;
    if (!p.causal) hi_key = min(hi_key, my_q + W - 1);
  }

  f32x16 dqacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqacc[dt] = (f32x16){};
  const float s2 = p.scale * kLog2e;
  const TrCoord trc(lane);

  // Byte offsets of this lane's operand reads in a tile (rows per K-step,
  // transposing reads per d-tile and row half), re-hidden from the optimizer
  // before use so that slot constants fold into the reads.
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
  auto rrow = [&](const __bf16* t, int ks) {
    return *(const bf16x8*)((const char*)t + roff[ks]);
  };
  auto rtr = [&](const __bf16* t, int j) {  // K-step j / DT, d-tile j % DT
    const char* b = (const char*)t + 16 * (j / DT) * D * 2;
    return cat4(lds_read_tr16(b + toff[2 * (j % DT)]), lds_read_tr16(b + toff[2 * (j % DT) + 1]));
  };

  f32x16 snx, dpnx;  // S^T and D - dP^T of the tile whose dS comes next
  bf16x8 dsop[2];
  // Mask, P and dS^T (negated) of tile t from snx, dpnx into dsop.
  auto ds_step = [&](int t) {
    const int kv0 = t * BC;
    bool need_mask = (kv0 + BC > N) || (wq0 + 32 > N);
    if (p.causal) need_mask |= kv0 + BC - 1 > wq0;
    if (W > 0) {
      need_mask |= wq0 + 31 - kv0 >= W;
      if (!p.causal) need_mask |= kv0 + BC - 1 - wq0 >= W;
    }
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 8 * (r >> 2) + 4 * h + (r & 3);
        snx[r] = (key > hi_key || key < lo_key || !q_ok) ? -__builtin_inff() : snx[r];
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = fast_exp2(fmaf(snx[e], s2, -Lb));
      dsop[e >> 3][e & 7] = (__bf16)(pv * dpnx[e]);
    }
  };

  // Prologue: K_0..K_2, V_0..V_2; S^T, D - dP^T and dS^T of tile 0.
  tile_load_lds<D, BC, NWV>(kh, head_bytes, t_lo * BC, sK0, w, lane);
  tile_load_lds<D, BC, NWV>(vh, head_bytes, t_lo * BC, sV0, w, lane);
  tile_load_lds<D, BC, NWV>(kh, head_bytes, (t_lo + 1) * BC, sK1, w, lane);
  tile_load_lds<D, BC, NWV>(vh, head_bytes, (t_lo + 1) * BC, sV1, w, lane);
  tile_load_lds<D, BC, NWV>(kh, head_bytes, (t_lo + 2) * BC, sK2, w, lane);
  tile_load_lds<D, BC, NWV>(vh, head_bytes, (t_lo + 2) * BC, sV2, w, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  snx = (f32x16){};
  dpnx = dp0;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    snx = mfma32(tile_row8<D>(sK0, n, 2 * ks + h), qop[ks], snx);
    dpnx = mfma32(tile_row8<D>(sV0, n, 2 * ks + h), doop[ks], dpnx);
  }
  ds_step(t_lo);

  auto end_half = [&]() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2));
    __builtin_amdgcn_s_barrier();
  };
  // Fetches of even half-step 2u: K_{u+3} and V_{u+3} into slot (u+3) % 4.
  auto fetch = [&](int u, __bf16* Kf, __bf16* Vf) {
    tile_load_lds<D, BC, NWV>(kh, head_bytes, (t_lo + u + 3) * BC, Kf, w, lane);
    tile_load_lds<D, BC, NWV>(vh, head_bytes, (t_lo + u + 3) * BC, Vf, w, lane);
  };
  // M(u): operand i of the 3 KS MFMAs is, by i % 3, a K row (S of tile
  // u+1), a V row (dP of tile u+1) or a transposed K_u pair (dQ, K-step and
  // d-tile (i / 3) / DT, (i / 3) % DT).
  bf16x8 opd[NM];
  auto issue = [&](int i, const __bf16* Kc, const __bf16* Kn, const __bf16* Vn) {
    const int j = i / 3;
    if (i % 3 == 0) opd[i] = rrow(Kn, j);
    else if (i % 3 == 1) opd[i] = rrow(Vn, j);
    else opd[i] = rtr(Kc, j);
  };
  auto prefetch = [&](const __bf16* Kc, const __bf16* Kn, const __bf16* Vn) {
    hide();
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) issue(i, Kc, Kn, Vn);
  };
  auto mstep = [&](const __bf16* Kc, const __bf16* Kn, const __bf16* Vn) {
    hide();
    f32x16 s = (f32x16){}, dp = dp0;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + AHEAD < NM) issue(i + AHEAD, Kc, Kn, Vn);
      const int j = i / 3;
      if (i % 3 == 0) s = mfma32(opd[i], qop[j], s);
      else if (i % 3 == 1) dp = mfma32(opd[i], doop[j], dp);
      else dqacc[j % DT] = mfma32(opd[i], dsop[j / DT], dqacc[j % DT]);
      __builtin_amdgcn_sched_barrier(0);
    }
    snx = s;
    dpnx = dp;
  };
  auto vstep = [&](int u, int Tg) {
    if (u >= 0 && u + 1 < Tg) ds_step(t_lo + u + 1);
  };

  int u = 0;
  if (lead) {
    const int Tg = p.causal ? min(T, (q0 + 32 * NG - 1) / BC - t_lo + 1) : T;
    prefetch(sK0, sK1, sV1);
    for (; u + 4 <= Tg; u += 4) {
      fetch(u, sK3, sV3);
      mstep(sK0, sK1, sV1);
      end_half();
      prefetch(sK1, sK2, sV2);
      vstep(u, Tg);
      end_half();
      fetch(u + 1, sK0, sV0);
      mstep(sK1, sK2, sV2);
      end_half();
      prefetch(sK2, sK3, sV3);
      vstep(u + 1, Tg);
      end_half();
      fetch(u + 2, sK1, sV1);
      mstep(sK2, sK3, sV3);
      end_half();
      prefetch(sK3, sK0, sV0);
      vstep(u + 2, Tg);
      end_half();
      fetch(u + 3, sK2, sV2);
      mstep(sK3, sK0, sV0);
      end_half();
      prefetch(sK0, sK1, sV1);
      vstep(u + 3, Tg);
      end_half();
    }
    if (u < Tg) {
      fetch(u, sK3, sV3);
      mstep(sK0, sK1, sV1);
      end_half();
      prefetch(sK1, sK2, sV2);
      vstep(u, Tg);
      end_half();
    }
    if (u + 1 < Tg) {
      fetch(u + 1, sK0, sV0);
      mstep(sK1, sK2, sV2);
      end_half();
      prefetch(sK2, sK3, sV3);
      vstep(u + 1, Tg);
      end_half();
    }
    if (u + 2 < Tg) {
      fetch(u + 2, sK1, sV1);
      mstep(sK2, sK3, sV3);
      end_half();
      prefetch(sK3, sK0, sV0);
      vstep(u + 2, Tg);
      end_half();
    }
    for (u += (u < Tg) + (u + 1 < Tg) + (u + 2 < Tg); u < T; ++u) {
      if (u % 4 == 0) fetch(u, sK3, sV3);
      else if (u % 4 == 1) fetch(u, sK0, sV0);
      else if (u % 4 == 2) fetch(u, sK1, sV1);
      else fetch(u, sK2, sV2);
      end_half();
      end_half();
    }
    end_half();
  } else {
    for (; u + 4 <= T; u += 4) {
      fetch(u, sK3, sV3);
      prefetch(sK0, sK1, sV1);
      vstep(u - 1, T);
      end_half();
      mstep(sK0, sK1, sV1);
      end_half();
      fetch(u + 1, sK0, sV0);
      prefetch(sK1, sK2, sV2);
      vstep(u, T);
      end_half();
      mstep(sK1, sK2, sV2);
      end_half();
      fetch(u + 2, sK1, sV1);
      prefetch(sK2, sK3, sV3);
      vstep(u + 1, T);
      end_half();
      mstep(sK2, sK3, sV3);
      end_half();
      fetch(u + 3, sK2, sV2);
      prefetch(sK3, sK0, sV0);
      vstep(u + 2, T);
      end_half();
      mstep(sK3, sK0, sV0);
      end_half();
    }
    if (u < T) {
      fetch(u, sK3, sV3);
      prefetch(sK0, sK1, sV1);
      vstep(u - 1, T);
      end_half();
      mstep(sK0, sK1, sV1);
      end_half();
    }
    if (u + 1 < T) {
      fetch(u + 1, sK0, sV0);
      prefetch(sK1, sK2, sV2);
      vstep(u, T);
      end_half();
      mstep(sK1, sK2, sV2);
      end_half();
    }
    if (u + 2 < T) {
      fetch(u + 2, sK1, sV1);
      prefetch(sK2, sK3, sV3);
      vstep(u + 1, T);
      end_half();
      mstep(sK2, sK3, sV3);
      end_half();
    }
    end_half();
  }
  __builtin_amdgcn_s_waitcnt(0);  // no fetch may land after the workgroup ends

  if (q_ok) {
    const size_t row = head + (size_t)my_q * D;
    const float qs = -p.scale;  // (dS negated)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(p.dq + row + 32 * dt + 8 * g + 4 * h) =
            (f32x4){dqacc[dt][4 * g] * qs, dqacc[dt][4 * g + 1] * qs,
                    dqacc[dt][4 * g + 2] * qs, dqacc[dt][4 * g + 3] * qs};
  }
}

static BwdKParams bwd_params(const BwdArgs& a, int tile_rows) {
  BwdKParams p;
  p.q = (const __bf16*)a.q;
  p.k = (const __bf16*)a.k;
  p.v = (const __bf16*)a.v;
  p.o = (const __bf16*)a.o;
  p.dout = (const __bf16*)a.dout;
  p.lse = a.lse;
  p.delta = a.delta;
  p.lse2 = a.lse2;
  p.H = a.H;
  p.Hkv = a.Hkv;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.N = a.N;
  p.scale = a.scale;
  p.causal = a.causal;
  p.window = a.window;
  p.n_tiles = (a.N + tile_rows - 1) / tile_rows;
  p.drop = make_dropout(a.drop);
  p.dk_part = a.dk_part;
  p.dv_part = a.dv_part;
  p.split = 1;
  return p;
}

constexpr int kBwdWaves = 4;
// Query rows per step of the dK/dV kernel.
template <int D>
constexpr int dkdv_qtile() { return D == 64 ? 32 : 64; }
// With dropout, 32-row steps: the keep bytes need registers that the 64-row
// step does not have to spare.
constexpr int kDropQTile = 32;

hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t stream) {
  const int rows = a.BH * a.N;
  if (a.d == 128) {
    constexpr int RPB = 256 / 16;
    hipLaunchKernelGGL((bwd_delta_kernel<128>), dim3((rows + RPB - 1) / RPB),
                       dim3(256), 0, stream, (const __bf16*)a.o,
                       (const __bf16*)a.dout, a.lse, a.delta, a.lse2, rows);
  } else {
    constexpr int RPB = 256 / 8;
    hipLaunchKernelGGL((bwd_delta_kernel<64>), dim3((rows + RPB - 1) / RPB),
                       dim3(256), 0, stream, (const __bf16*)a.o,
                       (const __bf16*)a.dout, a.lse, a.delta, a.lse2, rows);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream, const char** name) {
  BwdKParams p = bwd_params(a, 32 * kBwdWaves);
  // One workgroup per key block of every key/value head and share of its group.
  const int BHkv = a.BH / a.H * a.Hkv;
  p.split = a.no_split ? 1 : dkdv_split(BHkv, a.H / a.Hkv, a.N, a.d, a.causal);
  const dim3 grid((unsigned)(BHkv * p.n_tiles * p.split)), block(64 * kBwdWaves);
  const bool drop = a.drop.thresh > 0;
  constexpr int W = kBwdWaves;
  hipError_t e;
  if (a.d == 128 && drop)
    e = go<bwd_dkdv_kernel<128, W, kDropQTile, true>>(
        name, kname("attn::bwd_dkdv_kernel", 128, W, kDropQTile, true), grid, block, stream, p);
  else if (a.d == 128)
    e = go<bwd_dkdv_quad_kernel<128>>(name, kname("attn::bwd_dkdv_quad_kernel", 128), grid,
                                      dim3(512), stream, p);
  else if (drop)
    e = go<bwd_dkdv_kernel<64, W, kDropQTile, true>>(
        name, kname("attn::bwd_dkdv_kernel", 64, W, kDropQTile, true), grid, block, stream, p);
  else if (a.causal)
    e = go<bwd_dkdv_kernel<64, W, dkdv_qtile<64>(), false>>(
        name, kname("attn::bwd_dkdv_kernel", 64, W, dkdv_qtile<64>(), false), grid, block,
        stream, p);
  else {
    // d = 64 without dropout or causal mask: the ping-pong kernel, 256 keys
    // per workgroup (the same shares of the group, so the same workspace).
    // Under the causal mask its second group would compute four query tiles
    // its keys cannot see (measured 0.5-1.5 % slower), so causal launches keep
    // the kernel above.
    BwdKParams pp = bwd_params(a, 64 * W);
    pp.split = p.split;
    e = go<bwd_dkdv_pp_kernel<64, W>>(name, kname("attn::bwd_dkdv_pp_kernel", 64, W),
                                      dim3((unsigned)(BHkv * pp.n_tiles * pp.split)),
                                      dim3(2 * 64 * W), stream, pp);
  }
  if (name || e != hipSuccess) return e;
  if (p.split > 1) {
    const size_t n4 = (size_t)BHkv * a.N * a.d / 4;
    const unsigned sum_grid = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
    hipLaunchKernelGGL(bwd_share_sum_kernel, dim3(sum_grid), dim3(256), 0, stream,
                       (const f32x4*)a.dk_part, (f32x4*)a.dk, n4, p.split);
    hipLaunchKernelGGL(bwd_share_sum_kernel, dim3(sum_grid), dim3(256), 0, stream,
                       (const f32x4*)a.dv_part, (f32x4*)a.dv, n4, p.split);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream, const char** name) {
  const BwdKParams p = bwd_params(a, 32 * kBwdWaves);
  const dim3 grid((unsigned)(a.BH * p.n_tiles)), block(64 * kBwdWaves);
  const bool drop = a.drop.thresh > 0;
  constexpr int W = kBwdWaves;
  if (a.d == 128 && drop)
    return go<bwd_dq_kernel<128, W, 32, true>>(name, kname("attn::bwd_dq_kernel", 128, W, 32, true),
                                               grid, block, stream, p);
  if (a.d == 128) {
    const BwdKParams pp = bwd_params(a, 64 * W);
    return go<bwd_dq_pp_kernel<128, W>>(name, kname("attn::bwd_dq_pp_kernel", 128, W),
                                        dim3((unsigned)(a.BH * pp.n_tiles)), dim3(2 * 64 * W),
                                        stream, pp);
  }
  if (drop)
    return go<bwd_dq_kernel<64, W, 64, true>>(name, kname("attn::bwd_dq_kernel", 64, W, 64, true),
                                              grid, block, stream, p);
  return go<bwd_dq_kernel<64, W, 64, false>>(name, kname("attn::bwd_dq_kernel", 64, W, 64, false),
                                             grid, block, stream, p);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  hipError_t e = launch_bwd_dq(a, stream);
  if (e == hipSuccess) e = launch_bwd_dkdv(a, stream);
  return e;
}

}  // namespace attn

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
// Three launches on the caller's stream:
//  1. bwd_delta_kernel: D = rowsum(dO * O) (memory-bound, one pass);
//  2. bwd_dkdv_kernel: one workgroup per K/V block (the page's column-block
//     partition of the backward), K_j and V_j resident in VGPRs, looping over
//     the query blocks that can see them; dK_j and dV_j accumulate in VGPRs
//     and are written once;
//  3. bwd_dq_kernel: one workgroup per query block, Q_i, dO_i, L_i, D_i
//     resident, looping over the K/V blocks it sees; dQ_i accumulates in
//     VGPRs and is written once.
// Splitting dQ into its own pass recomputes S and dP there (two extra
// products per visible tile) but needs no atomics and no zeroed buffer, and
// the result is deterministic.
//
// gfx950 mapping.  In the dK/dV kernel each wave owns 32 keys and computes
// S = Q K^T with keys on the MFMA N side, so the C layout gives one key per
// lane and P, dS (bf16) are directly the B operands of dV^T += dO^T P and
// dK^T += Q^T dS; dO^T and Q^T are read from LDS with transposing reads in
// the C layout's row permutation.  The dQ kernel is the mirror image: S^T =
// K Q^T with one query per lane, and dQ^T += K^T dS^T with K^T read
// transposed from LDS.  Q/dO (dK/dV kernel) and K/V (dQ kernel) tiles are
// double-buffered in LDS with the same swizzle as the forward.
#include "attn_device.hpp"
#include "attn_kernels.hpp"

namespace attn {

__device__ __forceinline__ float bf16_lo(uint32_t x) {
  return __builtin_bit_cast(float, x << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t x) {
  return __builtin_bit_cast(float, x & 0xffff0000u);
}

// D_i = sum_k dO_ik O_ik over rows of d elements; D/8 threads per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const __bf16* o,
                                                        const __bf16* dout,
                                                        float* delta, int rows) {
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
  if (r < rows && c == 0) delta[r] = acc;
}

struct BwdKParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  int N;
  int n_tiles;
  float scale;
  int causal, window;
};

// ---------------------------------------------------------------- dK, dV
template <int D, int NW, int BQ>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_kernel(BwdKParams p) {
  constexpr int BKV = 32 * NW;  // keys per workgroup
  constexpr int NT = NW * 64;
  static_assert(BQ % 32 == 0 && BQ <= NT, "query tile");
  __shared__ __attribute__((aligned(16))) __bf16 sQ[2][BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 sdO[2][BQ * D];
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];
  __shared__ __attribute__((aligned(16))) float sD[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / p.n_tiles;
  const int kt = logical % p.n_tiles;  // low key blocks see the most queries
  const int N = p.N, W = p.window;
  const int k0 = kt * BKV;
  const int kw0 = k0 + 32 * w;
  const int my_k = kw0 + n;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc(p.q + head, head_bytes);
  const auto rk = make_rsrc(p.k + head, head_bytes);
  const auto rv = make_rsrc(p.v + head, head_bytes);
  const auto rdo = make_rsrc(p.dout + head, head_bytes);
  const float* lse = p.lse + (size_t)bh * N;
  const float* delta = p.delta + (size_t)bh * N;

  // K^T and V^T as B operands (lane = key, 8 consecutive d per K-step).
  bf16x8 kop[D / 16], vop[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint32_t off = (uint32_t)(my_k * D + 16 * ks + 8 * h) * 2u;
    kop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
    vop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dkacc[dt] = dvacc[dt] = (f32x16){};

  // Queries that can see any key of this block.
  const int k_last = min(k0 + BKV, N) - 1;
  int q_lo = p.causal ? k0 : 0, q_hi = N;
  if (W > 0) {
    q_lo = max(q_lo, k0 - W + 1);
    q_hi = min(q_hi, k_last + W);
  }
  const int t_lo = q_lo / BQ, t_hi = (q_hi + BQ - 1) / BQ;

  TileStage<D, BQ, NT> stQ, stO;
  float stL = 0.f, stD = 0.f;
  auto load_tile = [&](int t) {
    stQ.load(rq, t * BQ, tid);
    stO.load(rdo, t * BQ, tid);
    if (tid < BQ) {
      const int i = t * BQ + tid;
      stL = i < N ? lse[i] * kLog2e : 0.f;
      stD = i < N ? delta[i] : 0.f;
    }
  };
  auto store_tile = [&](int b) {
    stQ.store(sQ[b], tid);
    stO.store(sdO[b], tid);
    if (tid < BQ) {
      sL[b][tid] = stL;
      sD[b][tid] = stD;
    }
  };

  const float s2 = p.scale * kLog2e;
  const TrCoord trc(lane);
  if (t_lo < t_hi) {
    load_tile(t_lo);
    store_tile(0);
  }
  __syncthreads();

  int buf = 0;
  for (int t = t_lo; t < t_hi; ++t) {
    const bool has_next = t + 1 < t_hi;
    if (has_next) load_tile(t + 1);
    const int i0 = t * BQ;
    // Does any (query of this tile, key of this wave) pair survive the mask?
    bool active = kw0 < N;
    if (p.causal) active &= i0 + BQ - 1 >= kw0;
    if (W > 0) {
      active &= i0 - (kw0 + 31) < W;
      if (!p.causal) active &= kw0 - (i0 + BQ - 1) < W;
    }
    if (active) {
      const __bf16* Qs = sQ[buf];
      const __bf16* Os = sdO[buf];
      // S = Q K^T and dP = dO V^T (queries on M, this wave's keys on N).
      f32x16 sacc[BQ / 32], dpacc[BQ / 32];
#pragma unroll
      for (int mt = 0; mt < BQ / 32; ++mt) {
        sacc[mt] = dpacc[mt] = (f32x16){};
        const int r = 32 * mt + n;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          sacc[mt] = mfma32(tile_row8<D>(Qs, r, 2 * ks + h), kop[ks], sacc[mt]);
          dpacc[mt] = mfma32(tile_row8<D>(Os, r, 2 * ks + h), vop[ks], dpacc[mt]);
        }
      }
      bool need_mask = (i0 + BQ > N) || (kw0 + 32 > N);
      if (p.causal) need_mask |= i0 < kw0 + 31;
      if (W > 0) {
        need_mask |= (i0 + BQ - 1) - kw0 >= W;
        if (!p.causal) need_mask |= (kw0 + 31) - i0 >= W;
      }
      // P = exp(s S - L), dS = P (dP - D); rows are queries 32mt + 8g + 4h + 0..3.
      bf16x8 pop[BQ / 16], dsop[BQ / 16];
#pragma unroll
      for (int mt = 0; mt < BQ / 32; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qi = 32 * mt + 8 * g + 4 * h;
          const f32x4 Lb = *(const f32x4*)&sL[buf][qi];
          const f32x4 Dl = *(const f32x4*)&sD[buf][qi];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float sv = sacc[mt][r];
            if (need_mask) {
              const int qq = i0 + qi + e;
              if (!(qq < N && visible(qq, my_k, N, p.causal, W))) sv = -__builtin_inff();
            }
            const float pv = fast_exp2(fmaf(sv, s2, -Lb[e]));
            const float ds = pv * (dpacc[mt][r] - Dl[e]);
            pop[2 * mt + (r >> 3)][r & 7] = (__bf16)pv;
            dsop[2 * mt + (r >> 3)][r & 7] = (__bf16)ds;
          }
        }
      // dV^T += dO^T P, dK^T += Q^T dS (d on M, keys on N, queries contracted).
#pragma unroll
      for (int kk = 0; kk < BQ / 16; ++kk)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          dvacc[dt] = mfma32(tile_a_tr<D>(Os, trc, kk, dt), pop[kk], dvacc[dt]);
          dkacc[dt] = mfma32(tile_a_tr<D>(Qs, trc, kk, dt), dsop[kk], dkacc[dt]);
        }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  if (my_k < N) {
    const size_t row = head + (size_t)my_k * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        *(f32x4*)(p.dk + row + d0) =
            (f32x4){dkacc[dt][4 * g] * p.scale, dkacc[dt][4 * g + 1] * p.scale,
                    dkacc[dt][4 * g + 2] * p.scale, dkacc[dt][4 * g + 3] * p.scale};
        *(f32x4*)(p.dv + row + d0) = (f32x4){dvacc[dt][4 * g], dvacc[dt][4 * g + 1],
                                             dvacc[dt][4 * g + 2], dvacc[dt][4 * g + 3]};
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int D, int NW, int BC>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(BwdKParams p) {
  constexpr int BR = 32 * NW;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][BC * D];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / p.n_tiles;
  int qt = logical % p.n_tiles;
  if (p.causal) qt = p.n_tiles - 1 - qt;  // longest blocks first
  const int N = p.N, W = p.window;
  const int q0 = qt * BR;
  const int wq0 = q0 + 32 * w;
  const int my_q = wq0 + n;
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc(p.q + head, head_bytes);
  const auto rk = make_rsrc(p.k + head, head_bytes);
  const auto rv = make_rsrc(p.v + head, head_bytes);
  const auto rdo = make_rsrc(p.dout + head, head_bytes);

  // Q^T and dO^T as B operands (lane = query), L and D per lane.
  bf16x8 qop[D / 16], doop[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint32_t off = (uint32_t)(my_q * D + 16 * ks + 8 * h) * 2u;
    qop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    doop[ks] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
  }
  const bool q_ok = my_q < N;
  const float Lb = q_ok ? p.lse[(size_t)bh * N + my_q] * kLog2e : 0.f;
  const float Dl = q_ok ? p.delta[(size_t)bh * N + my_q] : 0.f;

  const int q_last = min(q0 + BR, N) - 1;
  int kv_lo = 0, kv_hi = N;
  if (p.causal) kv_hi = min(kv_hi, q_last + 1);
  if (W > 0) {
    kv_lo = max(0, q0 - W + 1);
    if (!p.causal) kv_hi = min(kv_hi, q_last + W);
  }
  const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;

  TileStage<D, BC, NT> stK, stV;
  auto load_tile = [&](int t) {
    stK.load(rk, t * BC, tid);
    stV.load(rv, t * BC, tid);
  };
  auto store_tile = [&](int b) {
    stK.store(smem[b][0], tid);
    stV.store(smem[b][1], tid);
  };

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dqacc[dt] = (f32x16){};
  const float s2 = p.scale * kLog2e;
  const TrCoord trc(lane);
  if (t_lo < t_hi) {
    load_tile(t_lo);
    store_tile(0);
  }
  __syncthreads();

  int buf = 0;
  for (int t = t_lo; t < t_hi; ++t) {
    const bool has_next = t + 1 < t_hi;
    if (has_next) load_tile(t + 1);
    const __bf16* Ks = smem[buf][0];
    const __bf16* Vs = smem[buf][1];
    const int kv0 = t * BC;
    bool active = wq0 < N;
    if (p.causal) active &= kv0 <= wq0 + 31;
    if (W > 0) {
      active &= wq0 - (kv0 + BC - 1) < W;
      if (!p.causal) active &= kv0 - (wq0 + 31) < W;
    }
    if (active) {
      // S^T = K Q^T and dP^T = V dO^T (keys on M, this wave's queries on N).
      f32x16 sacc[BC / 32], dpacc[BC / 32];
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt) {
        sacc[mt] = dpacc[mt] = (f32x16){};
        const int r = 32 * mt + n;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          sacc[mt] = mfma32(tile_row8<D>(Ks, r, 2 * ks + h), qop[ks], sacc[mt]);
          dpacc[mt] = mfma32(tile_row8<D>(Vs, r, 2 * ks + h), doop[ks], dpacc[mt]);
        }
      }
      bool need_mask = (kv0 + BC > N) || (wq0 + 32 > N);
      if (p.causal) need_mask |= kv0 + BC - 1 > wq0;
      if (W > 0) {
        need_mask |= wq0 + 31 - kv0 >= W;
        if (!p.causal) need_mask |= kv0 + BC - 1 - wq0 >= W;
      }
      bf16x8 dsop[BC / 16];
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sv = sacc[mt][r];
          if (need_mask) {
            const int key = kv0 + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
            if (!(q_ok && visible(my_q, key, N, p.causal, W))) sv = -__builtin_inff();
          }
          const float pv = fast_exp2(fmaf(sv, s2, -Lb));
          dsop[2 * mt + (r >> 3)][r & 7] = (__bf16)(pv * (dpacc[mt][r] - Dl));
        }
      // dQ^T += K^T dS^T (d on M, queries on N, keys contracted).
#pragma unroll
      for (int kk = 0; kk < BC / 16; ++kk)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          dqacc[dt] = mfma32(tile_a_tr<D>(Ks, trc, kk, dt), dsop[kk], dqacc[dt]);
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  if (q_ok) {
    const size_t row = head + (size_t)my_q * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        *(f32x4*)(p.dq + row + d0) =
            (f32x4){dqacc[dt][4 * g] * p.scale, dqacc[dt][4 * g + 1] * p.scale,
                    dqacc[dt][4 * g + 2] * p.scale, dqacc[dt][4 * g + 3] * p.scale};
      }
  }
}

static BwdKParams bwd_params(const BwdArgs& a, int tile_rows) {
  BwdKParams p;
  p.q = (const __bf16*)a.q;
  p.k = (const __bf16*)a.k;
  p.v = (const __bf16*)a.v;
  p.dout = (const __bf16*)a.dout;
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.N = a.N;
  p.scale = a.scale;
  p.causal = a.causal;
  p.window = a.window;
  p.n_tiles = (a.N + tile_rows - 1) / tile_rows;
  return p;
}

constexpr int kBwdWaves = 4;
constexpr int kBwdTile = 64;  // query rows (dK/dV kernel) or keys (dQ kernel) per step

hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t stream) {
  const int rows = a.BH * a.N;
  if (a.d == 128) {
    constexpr int RPB = 256 / 16;
    hipLaunchKernelGGL((bwd_delta_kernel<128>), dim3((rows + RPB - 1) / RPB),
                       dim3(256), 0, stream, (const __bf16*)a.o,
                       (const __bf16*)a.dout, a.delta, rows);
  } else {
    constexpr int RPB = 256 / 8;
    hipLaunchKernelGGL((bwd_delta_kernel<64>), dim3((rows + RPB - 1) / RPB),
                       dim3(256), 0, stream, (const __bf16*)a.o,
                       (const __bf16*)a.dout, a.delta, rows);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  const BwdKParams p = bwd_params(a, 32 * kBwdWaves);
  const dim3 grid((unsigned)(a.BH * p.n_tiles)), block(64 * kBwdWaves);
  if (a.d == 128)
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, kBwdWaves, kBwdTile>), grid, block, 0,
                       stream, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, kBwdWaves, kBwdTile>), grid, block, 0,
                       stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  const BwdKParams p = bwd_params(a, 32 * kBwdWaves);
  const dim3 grid((unsigned)(a.BH * p.n_tiles)), block(64 * kBwdWaves);
  if (a.d == 128)
    hipLaunchKernelGGL((bwd_dq_kernel<128, kBwdWaves, kBwdTile>), grid, block, 0,
                       stream, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<64, kBwdWaves, kBwdTile>), grid, block, 0,
                       stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  hipError_t e = launch_bwd_preprocess(a, stream);
  if (e == hipSuccess) e = launch_bwd_dkdv(a, stream);
  if (e == hipSuccess) e = launch_bwd_dq(a, stream);
  return e;
}

}  // namespace attn

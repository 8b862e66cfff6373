// attn_fwd.hip -- bf16 forward kernel for gfx950.
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
//    reductions plus one permlane32 swap, and the rescale factor is a
//    per-lane scalar.
//  * The probabilities P^T, converted to bf16 in place, are directly the B
//    operand of O^T += V_j^T P^T (d on the M side).  V_j^T is read from LDS
//    with ds_read_b64_tr_b16 using the key permutation of the C layout
//    (see attn_device.hpp), so nothing moves between lanes.
//  * Q_i^T stays in VGPRs for the whole K/V loop; K_j and V_j are
//    double-buffered in LDS: the next tile's global loads are issued before
//    the current tile's math and written to the other buffer after it.
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
#include "attn_device.hpp"
#include "attn_kernels.hpp"

namespace attn {

struct FwdKParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  void* o;
  float* lse;
  int N;
  int n_qtiles;
  float scale;
  int causal, window, out_f32;
};

template <int D, int NW, int BC>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(FwdKParams p) {
  constexpr int BR = 32 * NW;          // queries per workgroup
  constexpr int NT = NW * 64;          // threads per workgroup
  static_assert(BC % 32 == 0, "key tile is a multiple of 32");
  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][BC * D];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / p.n_qtiles;
  int qt = logical % p.n_qtiles;
  if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest blocks first
  const int N = p.N;
  const int q0 = qt * BR;
  const int wq0 = q0 + 32 * w;             // first query of this wave
  const int my_q = wq0 + n;                // this lane's query
  const size_t head = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto rq = make_rsrc(p.q + head, head_bytes);
  const auto rk = make_rsrc(p.k + head, head_bytes);
  const auto rv = make_rsrc(p.v + head, head_bytes);

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

  TileStage<D, BC, NT> stK, stV;
  auto load_tile = [&](int t) {
    stK.load(rk, t * BC, tid);
    stV.load(rv, t * BC, tid);
  };
  auto store_tile = [&](int b) {
    stK.store(smem[b][0], tid);
    stV.store(smem[b][1], tid);
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = (f32x16){};
  float m_run = kMaxInit, l_run = 0.f;
  const float s2 = p.scale * kLog2e;
  const float tau = 8.0f / s2;

  if (t_lo < t_hi) {
    load_tile(t_lo);
    store_tile(0);
  }
  __syncthreads();

  const TrCoord trc(lane);  // transposing-read coordinates of this lane

  int buf = 0;
  for (int t = t_lo; t < t_hi; ++t) {
    const bool has_next = t + 1 < t_hi;
    if (has_next) load_tile(t + 1);
    const __bf16* Ks = smem[buf][0];
    const __bf16* Vs = smem[buf][1];
    const int kv0 = t * BC;

    // ---- S^T = K_j Q_i^T (raw scores, fp32) ----
    f32x16 sacc[BC / 32];
#pragma unroll
    for (int mt = 0; mt < BC / 32; ++mt) {
      sacc[mt] = (f32x16){};
      const int r = 32 * mt + n;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        sacc[mt] = mfma32(tile_row8<D>(Ks, r, 2 * ks + h), qop[ks], sacc[mt]);
    }

    // ---- mask only on tiles that straddle a boundary (wave-uniform test) ----
    bool need_mask = kv0 + BC > N;
    if (p.causal) need_mask |= kv0 + BC - 1 > wq0;
    if (p.window > 0) {
      need_mask |= wq0 + 31 - kv0 >= p.window;
      if (!p.causal) need_mask |= kv0 + BC - 1 - wq0 >= p.window;
    }
    if (need_mask) {
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
          if (!visible(my_q, key, N, p.causal, p.window))
            sacc[mt][r] = -__builtin_inff();
        }
    }

    // ---- online softmax, one query per lane ----
    float mx = -__builtin_inff();
#pragma unroll
    for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
    mx = halves_max(mx);
    const float m_new = (mx > m_run + tau) ? mx : m_run;
    const float alpha = fast_exp2((m_run - m_new) * s2);
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    }
    const float mb = m_run * s2;
    bf16x8 pop[BC / 16];
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(sacc[mt][r], s2, -mb));
        lsum += e;
        pop[2 * mt + (r >> 3)][r & 7] = (__bf16)e;
      }
    l_run += lsum;

    // ---- O^T += V_j^T P^T ----
#pragma unroll
    for (int kk = 0; kk < BC / 16; ++kk)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        oacc[dt] = mfma32(tile_a_tr<D>(Vs, trc, kk, dt), pop[kk], oacc[dt]);

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue: O = O~ / l, L = ln 2 * (m s2 + log2 l) ----
  const float l_tot = halves_sum(l_run);
  if (my_q < N) {
    const float inv = 1.f / l_tot;
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

template <int D, int NW, int BC>
static hipError_t launch_fwd_cfg(const FwdArgs& a, hipStream_t stream) {
  FwdKParams p;
  p.q = (const __bf16*)a.q;
  p.k = (const __bf16*)a.k;
  p.v = (const __bf16*)a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.n_qtiles = (a.N + 32 * NW - 1) / (32 * NW);
  p.scale = a.scale;
  p.causal = a.causal;
  p.window = a.window;
  p.out_f32 = a.out_f32;
  const unsigned grid = (unsigned)(a.BH * p.n_qtiles);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BC>), dim3(grid), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_fwd_cfg<128, 4, 64>(a, stream);
  return launch_fwd_cfg<64, 4, 64>(a, stream);
}

}  // namespace attn

// attn_decode.hip -- a short block of queries against a long key sequence
// (decode), split over the keys, for gfx950.
//
// Method.  In decode one new query row per head meets every cached key: the
// work is one pass over K and V and the kernel is bound by HBM bandwidth
// (the FlashAttention-3 page's point on inference).  One query block per
// head is far too little parallelism, so the keys of each key/value head are
// cut into chunks; each chunk gives a partial result (O_c, L_c) for every
// query row with the online-softmax recurrence of the forward, and a second
// kernel merges the partials with the softmax decomposition of the FLASH-ATTN
// page ("Tiling and Recomputation"): L = ln sum_c e^{L_c} and
// O = sum_c e^{L_c - L} O_c.
//
// Queries.  The block of Nq queries is the last Nq positions of the Nk-key
// sequence (query row i sits at key position Nk - Nq + i); the masks apply to
// that position.  All G = H / Hkv query heads that share a key/value head are
// handled together: their G * Nq rows are the 32 query lanes of the MFMA N
// side (several row blocks of 32 when G * Nq > 32), so every K/V byte is read
// once per row block.
//
// gfx950 mapping.  Each wave owns one (key/value head, row block, chunk) and
// runs on its own, with no barrier: S^T = K_t Q^T on v_mfma_f32_32x32x16_bf16
// with K_t read from global memory straight into the A-operand registers
// (one 16-byte load per lane and K-step), V_t fetched by direct global->LDS
// loads into a wave-private pair of swizzled LDS slots and read transposed
// (ds_read_b64_tr_b16) as the A operand of O^T += V_t^T P^T, as in the
// forward.  Two tiles (16 KB) are in flight per wave; the plan below runs
// about three waves per CU, which keeps more than enough bytes outstanding
// to cover the HBM latency (more in flight reads slower, not faster).
#include <algorithm>

#include "attn_device.hpp"
#include "attn_kernels.hpp"

namespace attn {

struct DecKParams {
  const __bf16* q;  // [B*H*Nq][D]
  const __bf16* k;  // [B*Hkv][Nk][D]
  const __bf16* v;
  float* opart;     // [B*H*Nq][P][D] partial outputs (normalised)
  float* lpart;     // [B*H*Nq][P] partial log-sum-exp (natural log)
  uint32_t q_bytes;
  int H, Hkv, G, Nq, Nk;
  int R, RB;        // rows per key/value head (G * Nq) and row blocks of 32
  int P, CW, kmin;  // chunks, keys per chunk, first key any row sees
  float scale;
  int causal, window;
};

template <int D>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecKParams p) {
  constexpr int BC = 32, KS = D / 16, NW = 4;
  constexpr int VLOADS = (BC * D / 8) / 64;  // one wave fills a V tile alone
  constexpr int kTileLoads = KS + VLOADS;    // vector-memory ops per tile
  __shared__ __attribute__((aligned(16))) __bf16 sV[NW][2][BC * D];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, kept scalar
  const int h = lane >> 5, n = lane & 31;
  const int wpu = (p.P + NW - 1) / NW;  // workgroups per (key/value head, row block)
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = logical / wpu;
  const int pc = (logical % wpu) * NW + w;  // this wave's chunk
  if (pc >= p.P) return;                     // (no barrier in this kernel)
  const int bkv = unit / p.RB, rb = unit % p.RB;
  const int b = bkv / p.Hkv, hk = bkv % p.Hkv;

  // This lane's query row: head j of the group, row qi of the block.
  const int r = 32 * rb + n;
  const bool row_ok = r < p.R;
  const int j = row_ok ? r / p.Nq : 0, qi = row_ok ? r % p.Nq : 0;
  const int rg = ((b * p.H) + hk * p.G + j) * p.Nq + qi;  // global query row
  const int pos = p.Nk - p.Nq + qi;
  const auto rq = make_rsrc(p.q, p.q_bytes);
  bf16x8 qop[KS];  // rows past R read as zeros (offset past the buffer)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qop[ks] = __builtin_bit_cast(
        bf16x8, buf_load16(rq, row_ok ? (uint32_t)(rg * D + 16 * ks + 8 * h) * 2u
                                      : p.q_bytes));

  // Keys of this chunk, and the ones this row may see: [lo, hi].
  const int c0 = p.kmin + pc * p.CW, c1 = min(p.Nk, c0 + p.CW);
  int lo = 0, hi = p.Nk - 1;
  if (row_ok) {
    if (p.causal) hi = pos;
    if (p.window > 0) {
      lo = max(0, pos - p.window + 1);
      if (!p.causal) hi = min(hi, pos + p.window - 1);
    }
  }
  lo = max(lo, c0);
  hi = min(hi, c1 - 1);

  const size_t head = (size_t)bkv * p.Nk * D;
  const uint32_t head_bytes = (uint32_t)p.Nk * D * 2;
  const auto rk = make_rsrc(p.k + head, head_bytes);
  __bf16* slot0 = sV[w][0];
  __bf16* slot1 = sV[w][1];

  // K rows as the A operand: lane holds K[kv0 + n][16 ks + 8 h .. +7].
  auto load_tile = [&](int kv0, bf16x8* kb, __bf16* vs) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kb[ks] = __builtin_bit_cast(
          bf16x8, buf_load16(rk, (uint32_t)((kv0 + n) * D + 16 * ks + 8 * h) * 2u));
    tile_load_lds<D, BC, 1>(p.v + head, head_bytes, kv0, vs, 0, lane);
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = (f32x16){};
  float m_run = kMaxInit, l_run = 0.f;
  const float s2 = p.scale * kLog2e;
  const float tau = 8.0f / s2;
  const TrCoord trc(lane);

  auto step = [&](int kv0, const bf16x8* kb, const __bf16* vs) {
    f32x16 sacc = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc = mfma32(kb[ks], qop[ks], sacc);
    // Register r holds key kv0 + 8(r/4) + 4h + r%4.
    if (__ballot(kv0 < lo || kv0 + BC - 1 > hi)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kv0 + 8 * (e >> 2) + 4 * h + (e & 3);
        sacc[e] = (key < lo || key > hi) ? -__builtin_inff() : sacc[e];
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
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
    bf16x8 pop[2];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float x = fast_exp2(fmaf(sacc[e], s2, -mb));
      lsum += x;
      pop[e >> 3][e & 7] = (__bf16)x;
    }
    l_run += lsum;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        oacc[dt] = mfma32(tile_a_tr<D>(vs, trc, kk, dt), pop[kk], oacc[dt]);
  };

  // Two tiles in flight: tile t computes while tile t+1 lands; tile t+2 is
  // fetched into t's buffers once t is done with them.  Tiles past the
  // chunk read rows of the next chunk or, past Nk, zeros; they are never
  // used.
  const int T = (c1 - c0 + BC - 1) / BC;
  bf16x8 kb0[KS], kb1[KS];
  load_tile(c0, kb0, slot0);
  load_tile(c0 + BC, kb1, slot1);
  for (int t = 0; t < T; t += 2) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kTileLoads));
    step(c0 + t * BC, kb0, slot0);
    load_tile(c0 + (t + 2) * BC, kb0, slot0);
    if (t + 1 < T) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kTileLoads));
      step(c0 + (t + 1) * BC, kb1, slot1);
      load_tile(c0 + (t + 3) * BC, kb1, slot1);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // Partial result of this chunk: O_c = O~ / l and L_c = ln 2 (m s2 + log2 l);
  // a row that sees no key of the chunk gives O_c = 0 and L_c = -inf.
  const float l_tot = halves_sum(l_run);
  if (row_ok) {
    const bool any = l_tot > 0.f;
    const float inv = any ? 1.f / l_tot : 0.f;
    float* orow = p.opart + ((size_t)rg * p.P + pc) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * h;
        *(f32x4*)(orow + d0) = (f32x4){oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv,
                                       oacc[dt][4 * g + 2] * inv,
                                       oacc[dt][4 * g + 3] * inv};
      }
    if (h == 0)
      p.lpart[(size_t)rg * p.P + pc] =
          any ? (m_run * s2 + __builtin_amdgcn_logf(l_tot)) * kLn2 : -__builtin_inff();
  }
}

struct DecMergeParams {
  const float* opart;
  const float* lpart;
  void* o;
  float* lse;
  int P, out_f32;
};

// One workgroup of 256 threads per query row: L = ln sum_c e^{L_c} and
// O = sum_c e^{L_c - L} O_c.  The weights e^{L_c - L} are formed once in LDS;
// the 256 / D slices of threads then each sum every (256/D)-th partial for
// all D elements (coalesced rows of O_c) and the slices are added in LDS.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecMergeParams p) {
  constexpr int NT = 256, S = NT / D;
  __shared__ float sW[1024];
  __shared__ float sRed[NT];
  const int rg = blockIdx.x, tid = threadIdx.x;
  const float* L = p.lpart + (size_t)rg * p.P;
  // max_c L_c
  float m = -__builtin_inff();
  for (int c = tid; c < p.P; c += NT) {
    const float x = L[c];
    sW[c] = x;
    m = fmaxf(m, x);
  }
  sRed[tid] = m;
  __syncthreads();
  for (int k = NT / 2; k > 0; k >>= 1) {
    if (tid < k) sRed[tid] = fmaxf(sRed[tid], sRed[tid + k]);
    __syncthreads();
  }
  m = sRed[0];
  __syncthreads();
  // sum_c e^{L_c - m}
  float s = 0.f;
  for (int c = tid; c < p.P; c += NT)
    if (sW[c] != -__builtin_inff()) s += __expf(sW[c] - m);
  sRed[tid] = s;
  __syncthreads();
  for (int k = NT / 2; k > 0; k >>= 1) {
    if (tid < k) sRed[tid] += sRed[tid + k];
    __syncthreads();
  }
  const float lt = m + __logf(sRed[0]);
  for (int c = tid; c < p.P; c += NT)
    sW[c] = (sW[c] == -__builtin_inff()) ? 0.f : __expf(sW[c] - lt);
  __syncthreads();
  // slice sl sums partials sl, sl + S, ... for element d
  const int d = tid % D, sl = tid / D;
  const float* O = p.opart + (size_t)rg * p.P * D + d;
  float a0 = 0.f, a1 = 0.f;
  int c = sl;
  for (; c + S < p.P; c += 2 * S) {
    a0 = fmaf(sW[c], O[(size_t)c * D], a0);
    a1 = fmaf(sW[c + S], O[(size_t)(c + S) * D], a1);
  }
  if (c < p.P) a0 = fmaf(sW[c], O[(size_t)c * D], a0);
  __syncthreads();
  sRed[tid] = a0 + a1;
  __syncthreads();
  if (sl == 0) {
    float acc = sRed[d];
#pragma unroll
    for (int k = 1; k < S; ++k) acc += sRed[k * D + d];
    if (p.out_f32)
      ((float*)p.o)[(size_t)rg * D + d] = acc;
    else
      ((__bf16*)p.o)[(size_t)rg * D + d] = (__bf16)acc;
    if (d == 0 && p.lse) p.lse[rg] = lt;
  }
}

DecodePlan decode_plan(int B, int H, int Hkv, int Nq, int Nk, int window) {
  DecodePlan pl;
  pl.G = H / Hkv;
  pl.R = pl.G * Nq;
  pl.RB = (pl.R + 31) / 32;
  // Keys no row can see (in front of every window) are skipped.
  int kmin = 0;
  if (window > 0) kmin = std::max(0, Nk - Nq - window + 1);
  pl.kmin = kmin & ~31;
  const int span = Nk - pl.kmin;
  // About 768 waves in all (three per CU), chunks of at least 128 keys, at
  // most 1024 chunks.  Fewer, longer key streams read HBM faster than more
  // of them: at B4 H32 H_kv8 N_k 32768, 768 waves take 97 us, 1024 take 101,
  // 2048 take 107 and 4096 take 123 (the same holds for a plain streaming
  // read, which is fastest with few bytes in flight per CU).
  const long units = (long)B * Hkv * pl.RB;
  long want = (768 + units - 1) / units;
  if (want < 1) want = 1;
  int cw = (int)((span + want - 1) / want);
  cw = (cw + 31) & ~31;
  if (cw < 128) cw = 128;
  int P = (span + cw - 1) / cw;
  if (P > 1024) {
    cw = (((span + 1023) / 1024) + 31) & ~31;
    P = (span + cw - 1) / cw;
  }
  pl.CW = cw;
  pl.P = P;
  return pl;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const DecodePlan pl = decode_plan(a.B, a.H, a.Hkv, a.Nq, a.Nk, a.window);
  DecKParams p;
  p.q = (const __bf16*)a.q;
  p.k = (const __bf16*)a.k;
  p.v = (const __bf16*)a.v;
  p.opart = a.opart;
  p.lpart = a.lpart;
  p.q_bytes = (uint32_t)((size_t)a.B * a.H * a.Nq * a.d * 2);
  p.H = a.H;
  p.Hkv = a.Hkv;
  p.G = pl.G;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.R = pl.R;
  p.RB = pl.RB;
  p.P = pl.P;
  p.CW = pl.CW;
  p.kmin = pl.kmin;
  p.scale = a.scale;
  p.causal = a.causal;
  p.window = a.window;
  const unsigned grid = (unsigned)((long)a.B * a.Hkv * pl.RB * ((pl.P + 3) / 4));
  if (a.d == 128)
    hipLaunchKernelGGL((decode_split_kernel<128>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<64>), dim3(grid), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DecMergeParams m;
  m.opart = a.opart;
  m.lpart = a.lpart;
  m.o = a.o;
  m.lse = a.lse;
  m.P = pl.P;
  m.out_f32 = a.out_f32;
  const unsigned rows = (unsigned)((long)a.B * a.H * a.Nq);
  if (a.d == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), dim3(rows), dim3(256), 0, stream, m);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), dim3(rows), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace attn

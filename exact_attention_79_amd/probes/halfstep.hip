// halfstep -- what lengthens the forward's matrix half-step beyond the 16 x 32
// cycles of its MFMAs.  The ping-pong forward (the FLASH-ATTN page's
// FlashAttention-3 "Background" paragraph motivates overlapping the softmax
// with the GEMMs) alternates, on every SIMD, one wave issuing 16
// v_mfma_f32_32x32x16_bf16 whose A operands it reads from LDS three MFMAs
// ahead (a row read, then two transposing reads, in turn) with one wave
// doing the softmax's vector work, a barrier after every half-step, while
// the K and V tiles stream into LDS by global -> LDS copies.  This program
// rebuilds that half-step piece by piece, with the library's own LDS tile
// layout (attn_device.hpp), on every CU of the chip.
//
// Part 1: one MFMA-only wave and one vector-only wave per SIMD, no LDS:
// cycles per MFMA with the partner idle, issuing fma, or issuing the
// softmax's fma + exp2 + add, with the accumulators in VGPRs or in AGPRs.
// Part 2: waves 0-3 run matrix half-steps (operands from LDS, random bf16
// data), waves 4-7 a vector partner; with or without a barrier after every
// half-step, with or without the tile copies (every wave 2 x 1 KB per two
// half-steps into a three-slot ring, waited two half-steps later, as the
// forward does), with the partner idle or doing 16 fma + exp2 + add.
//
// Every wave times itself with s_memtime (core clock cycles); lane 0 of
// each wave writes its cycle count.  The counts are averaged over waves.
//
// Build: hipcc --offload-arch=gfx950 -O3 -std=c++17 -I exact_attention_79_amd/csrc
//        exact_attention_79_amd/probes/halfstep.hip -o <exe>
// (build.py does this and places the program next to this file).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "attn_device.hpp"

using namespace attn;

#define CHECK(x)                                                      \
  do {                                                                \
    hipError_t e_ = (x);                                              \
    if (e_ != hipSuccess) {                                           \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));    \
      return 1;                                                       \
    }                                                                 \
  } while (0)

constexpr int kCUs = 256;

// A bf16 value in [-2, 2) from a hash of i (random-looking operand data).
__device__ __forceinline__ __bf16 hashed_bf16(uint32_t i) {
  uint32_t x = i * 2654435761u + 12345u;
  x ^= x >> 15;
  x *= 2246822519u;
  x ^= x >> 13;
  return (__bf16)(((float)(x & 0xFFFF) / 32768.f - 1.f) * 2.f);
}

// ---- Part 1 ----

// VK: 0 idle partner, 1 fma, 2 fma + exp2 + add.  AG: accumulators in AGPRs.
template <int VK, int AG>
__global__ __launch_bounds__(512, 1) void coissue(uint64_t* out, int iters, int viters) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w < 4) {
    bf16x8 A, B;
    for (int i = 0; i < 8; ++i) {
      A[i] = hashed_bf16(blockIdx.x * 4096 + threadIdx.x * 8 + i);
      B[i] = hashed_bf16(77777 + threadIdx.x * 8 + i);
    }
    f32x16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
    __builtin_amdgcn_s_barrier();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if constexpr (AG == 0) {
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, a1, 0, 0, 0);
          a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, a2, 0, 0, 0);
          a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, a3, 0, 0, 0);
        } else {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(a0) : "v"(A), "v"(B));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(a1) : "v"(A), "v"(B));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(a2) : "v"(A), "v"(B));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(a3) : "v"(A), "v"(B));
        }
      }
    }
    // (AGPR results are read by the compiler's moves below: the last MFMAs
    // must have written them.)
    if constexpr (AG == 1) asm volatile("s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7");
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    float s = 0.f;
    for (int r = 0; r < 16; ++r) s += a0[r] + a1[r] + a2[r] + a3[r];
    if (lane == 0) out[blockIdx.x * 8 + w] = (c1 - c0) + (s == 12345.f);
  } else {
    float x[11];
    for (int i = 0; i < 8; ++i) x[i] = lane * 0.01f - i * 0.1f;
    x[8] = 0.999f;
    x[9] = -0.001f;
    x[10] = 0.f;
    __builtin_amdgcn_s_barrier();
    for (int it = 0; it < viters; ++it) {
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int c = m & 7;
        if constexpr (VK == 1) x[c] = __builtin_fmaf(x[c], x[8], x[9]);
        if constexpr (VK == 2) {
          x[c] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[c], x[8], x[9]));
          x[10] += x[c];
        }
      }
    }
    float s = x[10];
    for (int i = 0; i < 8; ++i) s += x[i];
    if (lane == 0) out[blockIdx.x * 8 + w] = (s == 12345.f);  // keeps the work
  }
}

template <int VK, int AG>
static int part1(uint64_t* d, uint64_t* h, const char* name, bool print) {
  const int iters = 8000, viters = VK == 0 ? 0 : VK == 1 ? 12000 : 4000;
  for (int rep = 0; rep < 2; ++rep)
    hipLaunchKernelGGL((coissue<VK, AG>), dim3(kCUs), dim3(512), 0, 0, d, iters, viters);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  CHECK(hipMemcpy(h, d, kCUs * 8 * sizeof(uint64_t), hipMemcpyDeviceToHost));
  double c = 0;
  for (int b = 0; b < kCUs; ++b)
    for (int w = 0; w < 4; ++w) c += (double)h[b * 8 + w];
  if (print) std::printf("| %s | %.1f |\n", name, c / (kCUs * 4) / (16.0 * iters));
  return 0;
}

// ---- Part 2 ----

template <int BAR, int COPY, int VW>
__global__ __launch_bounds__(512, 1) void halfsteps(uint64_t* out, const __bf16* src,
                                                    uint32_t src_bytes, int iters) {
  __shared__ __attribute__((aligned(16))) __bf16 tile[2 * 32 * 128];      // K rows, V rows
  __shared__ __attribute__((aligned(16))) __bf16 ring[3 * 8 * 1024];      // copy slots
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 2 * 32 * 128; i += 512) tile[i] = hashed_bf16(blockIdx.x * 8192 + i);
  __syncthreads();
  const auto rs = make_rsrc(src, src_bytes);
  const uint32_t nchunks = src_bytes / 1024;
  // Two 1 KB pieces per wave into slot it % 3 (source chunks past the end
  // of the buffer are never addressed: c + 1 < nchunks).
  auto copy = [&](int it) {
    if constexpr (COPY) {
      const uint32_t c = ((uint32_t)(blockIdx.x * 97 + it) * 16u + (uint32_t)w * 2u) % (nchunks - 1);
      __bf16* dst = ring + (it % 3) * 8192 + w * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)dst, 16, (int)(c * 1024u + lane * 16u), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + 512), 16,
                                               (int)(c * 1024u + 1024u + lane * 16u), 0, 0, 0);
    }
  };
  auto end_half = [&]() {
    if constexpr (BAR) {
      if constexpr (COPY) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2));
      __builtin_amdgcn_s_barrier();
    }
  };
  __syncthreads();
  uint64_t c0 = 0, c1 = 0;
  float keep = 0.f;
  if (w < 4) {
    const int n = lane & 31, h = lane >> 5;
    const TrCoord trc(lane);
    bf16x8 B;
    for (int i = 0; i < 8; ++i) B[i] = hashed_bf16(99991 + lane * 8 + i);
    uint32_t roff[8], toff[8];
    for (int ks = 0; ks < 8; ++ks) roff[ks] = (uint32_t)tile_off<128>(n, 2 * ks + h) * 2u;
    for (int dt = 0; dt < 4; ++dt)
      for (int x = 0; x < 2; ++x) {
        const int r = trc.row + 8 * x, col = 32 * dt + trc.col;
        toff[2 * dt + x] = 8192u + (uint32_t)(tile_off<128>(r, col >> 3) + (col & 7)) * 2u;
      }
    bf16x8 op[16];
    auto rd = [&](int i) {  // operand i: a K row read (even) or two transposing V reads (odd)
      const char* b = (const char*)tile;
      const int j = i >> 1;
      if (i & 1) {
        const char* bb = b + 16 * (j / 4) * 128 * 2;
        op[i] = cat4(lds_read_tr16(bb + toff[2 * (j % 4)]), lds_read_tr16(bb + toff[2 * (j % 4) + 1]));
      } else {
        op[i] = *(const bf16x8*)(b + roff[j]);
      }
    };
    f32x16 acc[5] = {};
#pragma unroll
    for (int i = 0; i < 3; ++i) rd(i);
    c0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
      if (it % 2 == 0) copy(it / 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(roff[i]), "+v"(toff[i]));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        rd((i + 3) & 15);
        // Score-like products chain on one accumulator, P V-like ones
        // rotate over four, as in the forward.
        if (i & 1) acc[(i >> 1) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], B, acc[(i >> 1) & 3], 0, 0, 0);
        else acc[4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], B, acc[4], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      end_half();
    }
    c1 = __builtin_amdgcn_s_memtime();
    for (int j = 0; j < 5; ++j)
      for (int r = 0; r < 16; ++r) keep += acc[j][r];
  } else {
    float x[17];
    for (int i = 0; i < 16; ++i) x[i] = lane * 0.01f - i * 0.1f;
    x[16] = 0.f;
    c0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
      if (it % 2 == 0) copy(it / 2);
      if constexpr (VW) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          x[m] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[m], 0.999f, -0.001f));
          x[16] += x[m];
        }
      }
      end_half();
    }
    c1 = __builtin_amdgcn_s_memtime();
    keep = x[16];
  }
  __builtin_amdgcn_s_waitcnt(0);  // every copy has landed before the wave ends
  if (lane == 0) out[blockIdx.x * 8 + w] = (c1 - c0) + (keep == 12345.f);
}

template <int BAR, int COPY, int VW>
static int part2(uint64_t* d, uint64_t* h, const __bf16* src, uint32_t bytes, const char* name) {
  const int iters = 4000;
  for (int rep = 0; rep < 2; ++rep)
    hipLaunchKernelGGL((halfsteps<BAR, COPY, VW>), dim3(kCUs), dim3(512), 0, 0, d, src, bytes, iters);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  CHECK(hipMemcpy(h, d, kCUs * 8 * sizeof(uint64_t), hipMemcpyDeviceToHost));
  double cm = 0, cv = 0;
  for (int b = 0; b < kCUs; ++b)
    for (int w = 0; w < 8; ++w) (w < 4 ? cm : cv) += (double)h[b * 8 + w];
  cm /= kCUs * 4;
  cv /= kCUs * 4;
  std::printf("| %s | %.1f | %.0f | %.0f |\n", name, cm / (16.0 * iters), cm / iters, cv / iters);
  return 0;
}

int main() {
  uint64_t* d = nullptr;
  __bf16* src = nullptr;
  const uint32_t bytes = 256u << 20;
  CHECK(hipMalloc(&d, kCUs * 8 * sizeof(uint64_t)));
  CHECK(hipMalloc(&src, bytes));
  CHECK(hipMemset(src, 0x3c, bytes));
  uint64_t* h = (uint64_t*)std::malloc(kCUs * 8 * sizeof(uint64_t));
  if (!h) return 1;
  int e = 0;
  // The clock ramps up over the first few hundred milliseconds; one untimed
  // pass of part 1 first.
  for (int pass = 0; pass < 2; ++pass) {
    const bool print = pass == 1;
    if (print)
      std::printf("Part 1: cycles per MFMA of a wave issuing only MFMAs, with a vector-only partner wave on its SIMD\n\n"
                  "| partner, accumulators | cycles per MFMA |\n|---|---|\n");
    e |= part1<0, 0>(d, h, "idle, VGPRs", print);
    e |= part1<0, 1>(d, h, "idle, AGPRs", print);
    e |= part1<1, 0>(d, h, "fma, VGPRs", print);
    e |= part1<1, 1>(d, h, "fma, AGPRs", print);
    e |= part1<2, 0>(d, h, "fma + exp2 + add, VGPRs", print);
    e |= part1<2, 1>(d, h, "fma + exp2 + add, AGPRs", print);
  }
  std::printf("\nPart 2: matrix half-steps of 16 MFMAs with LDS operands (waves 0-3) and a partner (waves 4-7)\n\n"
              "| variant | cycles per MFMA | matrix wave cycles per half-step | partner cycles per half-step |\n"
              "|---|---|---|---|\n");
  e |= part2<0, 0, 1>(d, h, src, bytes, "no barrier, no copies, softmax-like partner");
  e |= part2<1, 0, 0>(d, h, src, bytes, "barrier, no copies, idle partner");
  e |= part2<1, 0, 1>(d, h, src, bytes, "barrier, no copies, softmax-like partner");
  e |= part2<1, 1, 0>(d, h, src, bytes, "barrier, copies, idle partner");
  e |= part2<1, 1, 1>(d, h, src, bytes, "barrier, copies, softmax-like partner");
  (void)hipFree(d);
  (void)hipFree(src);
  std::free(h);
  return e;
}

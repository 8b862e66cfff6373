// valu_rates -- measures what the vector work of the fp8 forward costs on the
// SIMD: the issue time of each vector instruction kind that forming the
// e4m3 weights uses (fma, add, exp2, the two f32 -> e4m3 converts and the
// e4m3 -> f32 convert), alone at 1, 2 and 4 waves per SIMD, and how much of
// that work overlaps the fp8 and bf16 matrix instructions when a wave issues
// both (the question the FLASH-ATTN page's FlashAttention-3 "Background"
// paragraph raises: fp8 doubles the matrix rate but not the exponential
// rate).
//
// Part 1: every wave runs 16 x ITERS instructions of one kind over eight
// independent register chains; the time per instruction and SIMD is the
// kernel time / (instructions per wave x waves per SIMD).
// Part 2: every bundle is one MFMA (four accumulators in rotation) followed
// by NV vector instructions of one kind on independent registers; the time
// per MFMA and SIMD shows how many of them the MFMA hides.
//
// One workgroup of four waves per CU per 256 workgroups (one wave per SIMD
// per 256).  Every lane writes one float of its own; no other memory.
//
// Build: hipcc --offload-arch=gfx950 -O3 exact_attention_79_amd/probes/valu_rates.hip -o <exe>
// (build.py does this and places the program next to this file).
#include <hip/hip_runtime.h>

#include <cstdio>

#define CHECK(x)                                                      \
  do {                                                                \
    hipError_t e_ = (x);                                              \
    if (e_ != hipSuccess) {                                           \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));    \
      return false;                                                   \
    }                                                                 \
  } while (0)

typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

enum Kind { FMA, ADD, EXP2, CVT_PK_FP8, CVT_SCALEF32_PK_FP8, CVT_PK_F32_FP8 };
static const char* kind_name(int k) {
  switch (k) {
    case FMA: return "v_fma_f32";
    case ADD: return "v_add_f32";
    case EXP2: return "v_exp_f32";
    case CVT_PK_FP8: return "v_cvt_pk_fp8_f32";
    case CVT_SCALEF32_PK_FP8: return "v_cvt_scalef32_pk_fp8_f32";
    default: return "v_cvt_pk_f32_fp8 (+ v_add_u32)";
  }
}

// One instruction of kind K on chain c (x and y are the eight chains).
template <int K>
__device__ __forceinline__ void op(float* x, int* y, int c) {
  if constexpr (K == FMA) x[c] = __builtin_fmaf(x[c], 1.0001f, 0.5f);
  if constexpr (K == ADD) x[c] = x[c] + x[(c + 3) & 7];
  if constexpr (K == EXP2) x[c] = __builtin_amdgcn_exp2f(x[c]);
  if constexpr (K == CVT_PK_FP8) y[c] = __builtin_amdgcn_cvt_pk_fp8_f32(x[c], x[(c + 1) & 7], y[c], false);
  if constexpr (K == CVT_SCALEF32_PK_FP8) {
    v2i16 t = __builtin_bit_cast(v2i16, y[c]);
    t = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(t, x[c], x[(c + 1) & 7], 0.0625f, false);
    y[c] = __builtin_bit_cast(int, t);
  }
  if constexpr (K == CVT_PK_F32_FP8) {
    const auto h = __builtin_amdgcn_cvt_pk_f32_fp8(y[c], false);
    x[c] = h[0];
    y[c] += __builtin_bit_cast(int, h[1]);
  }
}

template <int K>
__global__ __launch_bounds__(256, 1) void vector_only(float* out, int iters, float a0) {
  float x[8];
  int y[8];
  for (int i = 0; i < 8; ++i) {
    x[i] = a0 + threadIdx.x * 0.01f + i;
    y[i] = threadIdx.x + i;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 16; ++m) op<K>(x, y, m & 7);
  }
  float s = 0;
  for (int i = 0; i < 8; ++i) s += x[i] + (float)y[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// MF: 0 = v_mfma_f32_32x32x16_bf16, 1 = v_mfma_scale_f32_32x32x64_f8f6f4.
template <int MF, int NV, int K>
__global__ __launch_bounds__(256, 1) void matrix_and_vector(float* out, int iters, float a0) {
  f32x16 acc[4];
  for (int i = 0; i < 4; ++i) acc[i] = (f32x16){};
  bf16x8 A, B;
  i32x8 A8, B8;
  for (int i = 0; i < 8; ++i) {
    A[i] = (__bf16)(threadIdx.x * 0.001f + i);
    B[i] = (__bf16)(i * 0.5f);
    A8[i] = 0x38383838 + i;
    B8[i] = 0x30303030 + (int)threadIdx.x;
  }
  float x[8];
  int y[8];
  for (int i = 0; i < 8; ++i) {
    x[i] = a0 + threadIdx.x + i;
    y[i] = i;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if constexpr (MF == 0)
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[m & 3], 0, 0, 0);
      else
        acc[m & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A8, B8, acc[m & 3], 0, 0, 0,
                                                                    127, 0, 127);
#pragma unroll
      for (int v = 0; v < NV; ++v) op<K>(x, y, v & 7);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0;
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  for (int i = 0; i < 8; ++i) s += x[i] + (float)y[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Average time of one launch after one untimed launch, in ms.
template <typename F>
static bool time_ms(F launch, float* ms) {
  launch();
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0));
  launch();
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  CHECK(hipEventElapsedTime(ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return true;
}

constexpr int kCUs = 256;

template <int K>
static bool part1(float* out) {
  const int iters = 4000;
  std::printf("| %s |", kind_name(K));
  for (int wps : {1, 2, 4}) {
    const int grid = kCUs * wps;
    float ms;
    if (!time_ms([&] { hipLaunchKernelGGL(vector_only<K>, dim3(grid), dim3(256), 0, 0, out, iters, 0.1f); }, &ms))
      return false;
    std::printf(" %.2f |", ms * 1e6 / (16.0 * iters) / wps);
  }
  std::printf("\n");
  return true;
}

template <int MF, int NV, int K>
static bool part2(float* out) {
  const int iters = 1000;
  std::printf("| %s | %d %s |", MF ? "fp8 32x32x64 (scaled)" : "bf16 32x32x16", NV, kind_name(K));
  for (int wps : {1, 2}) {
    const int grid = kCUs * wps;
    float ms;
    if (!time_ms([&] {
          hipLaunchKernelGGL((matrix_and_vector<MF, NV, K>), dim3(grid), dim3(256), 0, 0, out, iters, 0.1f);
        }, &ms))
      return false;
    std::printf(" %.1f |", ms * 1e6 / (16.0 * iters) / wps);
  }
  std::printf("\n");
  return true;
}

int main() {
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)kCUs * 4 * 256 * sizeof(float)) != hipSuccess) return 1;
  bool ok = true;
  std::printf("Part 1: ns per instruction per SIMD (waves per SIMD: 1, 2, 4)\n\n");
  std::printf("| instruction | 1 | 2 | 4 |\n|---|---|---|---|\n");
  ok = ok && part1<FMA>(out) && part1<ADD>(out) && part1<EXP2>(out) && part1<CVT_PK_FP8>(out) &&
       part1<CVT_SCALEF32_PK_FP8>(out) && part1<CVT_PK_F32_FP8>(out);
  std::printf("\nPart 2: ns per MFMA per SIMD with NV vector instructions after each (waves per SIMD: 1, 2)\n\n");
  std::printf("| MFMA | vector work per MFMA | 1 | 2 |\n|---|---|---|---|\n");
  ok = ok && part2<0, 0, FMA>(out) && part2<0, 8, FMA>(out) && part2<0, 16, FMA>(out);
  ok = ok && part2<1, 0, FMA>(out) && part2<1, 8, FMA>(out) && part2<1, 16, FMA>(out) &&
       part2<1, 24, FMA>(out) && part2<1, 8, EXP2>(out) && part2<1, 8, CVT_PK_FP8>(out);
  (void)hipFree(out);
  return ok ? 0 : 1;
}

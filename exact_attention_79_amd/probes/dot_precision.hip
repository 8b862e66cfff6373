// dot_precision -- measures how exactly the matrix cores sum the 64 products
// of one score-sized dot product: v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3
// operands, one instruction per 64 products) against
// v_mfma_f32_32x32x16_bf16 (the same e4m3 values widened to bf16, which holds
// them exactly; four instructions per 64 products, fp32 accumulator).  The
// question is the fp8 forward's: the FLASH-ATTN page's FlashAttention-3
// summary runs both products of the attention forward in FP8, and inputs
// with outlier channels make one product of a score dominate the others.
//
// One wave computes C = A B^T for A, B: 32 x 64 e4m3 codes; the host compares
// every element with the exact sum of the decoded products and reports the
// largest absolute error and the largest error / sum_k |a_k b_k|, over 100
// draws of each operand pattern:
//   small     64 products of codes in 2^-4 .. 2^1 (no product dominates)
//   big+small one product of codes in 128 .. 240, the other 63 as above
//   big alone the big product, the other 63 zero
//   workload  rows of the fp8 workload: N(0,1) values with channel 17
//             scaled by 10, quantised with one scale (amax / 448)
//
// Build: hipcc --offload-arch=gfx950 -O3 exact_attention_79_amd/probes/dot_precision.hip -o <exe>
// (build.py does this and places the program next to this file).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#define CHECK(x)                                                      \
  do {                                                                \
    hipError_t e_ = (x);                                              \
    if (e_ != hipSuccess) {                                           \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));    \
      return 1;                                                       \
    }                                                                 \
  } while (0)

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// MODE 0: one fp8 MFMA over the 64 products; MODE 1: four bf16 MFMAs.
// Lane (n, h) holds row n of A and of B; the C layout puts register r of lane
// (n, h) at row 8 (r / 4) + 4 h + r % 4 of A, column n.
template <int MODE>
__global__ void dots(const uint8_t* A, const uint8_t* B, float* C) {
  const int lane = threadIdx.x, n = lane & 31, h = lane >> 5;
  f32x16 c = {};
  if constexpr (MODE == 0) {
    i32x8 a, b;  // k = 32 h .. 32 h + 31
    for (int i = 0; i < 8; ++i) {
      a[i] = *(const int*)(A + n * 64 + 32 * h + 4 * i);
      b[i] = *(const int*)(B + n * 64 + 32 * h + 4 * i);
    }
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  } else {
    for (int s = 0; s < 4; ++s) {  // K-step s: k = 16 s + 8 h .. +7
      bf16x8 a, b;
      for (int i = 0; i < 8; i += 2) {
        const int o = n * 64 + 16 * s + 8 * h + i;
        const int wa = A[o] | (A[o + 1] << 8), wb = B[o] | (B[o + 1] << 8);
        const bf16x2 pa = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wa, 1.f, false);
        const bf16x2 pb = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wb, 1.f, false);
        a[i] = pa[0], a[i + 1] = pa[1], b[i] = pb[0], b[i + 1] = pb[1];
      }
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
  }
  for (int r = 0; r < 16; ++r) C[(8 * (r / 4) + 4 * h + r % 4) * 32 + n] = c[r];
}

// OCP e4m3 (bias 7, no infinities, 0x7f / 0xff NaN).
static double e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  const double v = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

// Nearest e4m3 code of x (|x| <= 448), by search over the 127 positive codes.
static uint8_t e4m3_code(double x) {
  const double ax = std::fabs(x);
  int best = 0;
  for (int c = 1; c < 127; ++c)
    if (std::fabs(e4m3_value((uint8_t)c) - ax) < std::fabs(e4m3_value((uint8_t)best) - ax)) best = c;
  return (uint8_t)(best | (x < 0 ? 0x80 : 0));
}

int main() {
  std::mt19937 rng(7);
  std::uniform_int_distribution<int> u8(0, 255);
  std::normal_distribution<double> nrm(0.0, 1.0);
  auto small = [&]() { return (uint8_t)((u8(rng) & 0x87) | ((3 + u8(rng) % 6) << 3)); };  // 2^-4 .. 2^1 (x 1.875)
  auto big = [&]() { return (uint8_t)((u8(rng) & 0x80) | 0x70 | (u8(rng) & 7)); };       // 128 .. 240
  uint8_t *dA, *dB;
  float* dC;
  CHECK(hipMalloc(&dA, 32 * 64));
  CHECK(hipMalloc(&dB, 32 * 64));
  CHECK(hipMalloc(&dC, 32 * 32 * sizeof(float)));
  std::vector<uint8_t> A(32 * 64), B(32 * 64);
  std::vector<float> C(32 * 32);
  const char* pats[4] = {"small", "big+small", "big alone", "workload"};
  std::printf("| operands | fp8 MFMA: max abs err | max err / sum|ab| | bf16 MFMA: max abs err | max err / sum|ab| |\n");
  std::printf("|---|---|---|---|---|\n");
  for (int pat = 0; pat < 4; ++pat) {
    double worst[2] = {0, 0}, worst_rel[2] = {0, 0};
    for (int t = 0; t < 100; ++t) {
      if (pat < 3) {
        for (int r = 0; r < 32; ++r)
          for (int k = 0; k < 64; ++k) {
            const bool at_big = k == (t + r) % 64;
            A[r * 64 + k] = at_big && pat > 0 ? big() : pat == 2 ? 0 : small();
            B[r * 64 + k] = at_big && pat > 0 ? big() : pat == 2 ? 0 : small();
          }
      } else {
        std::vector<double> x(2 * 32 * 64);
        double amax = 0;
        for (size_t i = 0; i < x.size(); ++i) {
          x[i] = nrm(rng) * ((i % 64) == 17 ? 10.0 : 1.0);
          amax = std::fmax(amax, std::fabs(x[i]));
        }
        for (int i = 0; i < 32 * 64; ++i) {
          A[i] = e4m3_code(x[i] / amax * 448.0);
          B[i] = e4m3_code(x[32 * 64 + i] / amax * 448.0);
        }
      }
      CHECK(hipMemcpy(dA, A.data(), A.size(), hipMemcpyHostToDevice));
      CHECK(hipMemcpy(dB, B.data(), B.size(), hipMemcpyHostToDevice));
      for (int mode = 0; mode < 2; ++mode) {
        if (mode == 0) hipLaunchKernelGGL(dots<0>, dim3(1), dim3(64), 0, 0, dA, dB, dC);
        else hipLaunchKernelGGL(dots<1>, dim3(1), dim3(64), 0, 0, dA, dB, dC);
        CHECK(hipGetLastError());
        CHECK(hipMemcpy(C.data(), dC, C.size() * sizeof(float), hipMemcpyDeviceToHost));
        for (int i = 0; i < 32; ++i)
          for (int j = 0; j < 32; ++j) {
            double ex = 0, ab = 0;
            for (int k = 0; k < 64; ++k) {
              const double p = e4m3_value(A[i * 64 + k]) * e4m3_value(B[j * 64 + k]);
              ex += p;
              ab += std::fabs(p);
            }
            const double err = std::fabs(C[i * 32 + j] - ex);
            worst[mode] = std::fmax(worst[mode], err);
            if (ab > 0) worst_rel[mode] = std::fmax(worst_rel[mode], err / ab);
          }
      }
    }
    std::printf("| %s | %.4g | %.3g | %.4g | %.3g |\n", pats[pat], worst[0], worst_rel[0], worst[1],
                worst_rel[1]);
  }
  CHECK(hipFree(dA));
  CHECK(hipFree(dB));
  CHECK(hipFree(dC));
  return 0;
}

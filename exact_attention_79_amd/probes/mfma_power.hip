// mfma_power -- how fast the matrix cores run when they do nothing else, and
// at what clock: a loop of v_mfma_f32_32x32x16_bf16 (and of the fp16 and
// fp8 forms) on every SIMD of the chip, with operands of random bits or of
// constant values.  The question is what bounds the attention kernels (the
// FLASH-ATTN page's FlashAttention-3 "Background" paragraph compares the
// GEMM rate with the rest of the work): if the MFMAs alone cannot reach the
// nominal 2.4 GHz peak with random data, the chip's power, not the kernels'
// issue, sets the ceiling.
//
// Each wave keeps four independent accumulators and issues 16 MFMAs per
// loop iteration on operands held in registers (loaded once from a buffer of
// random bits or of one constant); one workgroup of WPS x 4 waves per CU.
// Lane 0 of every workgroup's first wave reads s_memtime (core clock cycles)
// and s_memrealtime (a constant 100 MHz counter) before and after its loop,
// which gives the core clock the loop ran at; the host times the launch
// with events and reports TFLOP/s, the fraction of the nominal peak and
// the clock.
//
// Build: hipcc --offload-arch=gfx950 -O3 exact_attention_79_amd/probes/mfma_power.hip -o <exe>
// (build.py does this and places the program next to this file).
#include <hip/hip_runtime.h>

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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCUs = 256;

// KIND 0: bf16 32x32x16; 1: fp16 32x32x16; 2: fp8 (e4m3) 32x32x64, scaled form.
// src: 32 words per lane (the A and B operands of four MFMAs).
// clk: per workgroup, {memtime start, memtime end, realtime start, realtime end}.
template <int KIND>
__global__ __launch_bounds__(512) void mfma_loop(const uint32_t* src, float* out,
                                                   unsigned long long* clk, int iters) {
  const int lane = threadIdx.x & 63;
  const uint32_t* s = src + ((blockIdx.x * blockDim.x + threadIdx.x) & 4095) * 32;
  u32x4 a[4], b[4];
  for (int i = 0; i < 4; ++i) {
    a[i] = (u32x4){s[8 * i], s[8 * i + 1], s[8 * i + 2], s[8 * i + 3]};
    b[i] = (u32x4){s[8 * i + 4], s[8 * i + 5], s[8 * i + 6], s[8 * i + 7]};
  }
  f32x16 acc[4];
  for (int i = 0; i < 4; ++i) acc[i] = (f32x16){};
  // fp8 operands: 32 codes per lane, made once from the same words.
  i32x8 fa[4], fb[4];
  for (int i = 0; i < 4; ++i) {
    fa[i] = (i32x8){(int)a[i][0], (int)a[i][1], (int)a[i][2], (int)a[i][3],
                    (int)b[i][0], (int)b[i][1], (int)b[i][2], (int)b[i][3]};
    fb[i] = (i32x8){(int)b[i][0], (int)b[i][1], (int)b[i][2], (int)b[i][3],
                    (int)a[i][0], (int)a[i][1], (int)a[i][2], (int)a[i][3]};
  }
  const bool timer = threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int i = m & 3;
      if constexpr (KIND == 0)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                          __builtin_bit_cast(bf16x8, b[i]),
                                                          acc[i], 0, 0, 0);
      else if constexpr (KIND == 1)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[i]),
                                                         __builtin_bit_cast(f16x8, b[i]),
                                                         acc[i], 0, 0, 0);
      else
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[i], acc[i], 0, 0, 0,
                                                                  127, 0, 127);
    }
  }
  if (timer) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clk[4 * blockIdx.x + 0] = t0;
    clk[4 * blockIdx.x + 1] = t1;
    clk[4 * blockIdx.x + 2] = r0;
    clk[4 * blockIdx.x + 3] = r1;
  }
  float sum = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) sum += acc[i][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
  (void)lane;
}

struct Run {
  double ms, tflops, ghz;
};

template <int KIND>
static bool run(const uint32_t* src, float* out, unsigned long long* clk, int wps, int iters,
                Run* r) {
  const int threads = 64 * 4 * wps;
  auto launch = [&] {
    hipLaunchKernelGGL(mfma_loop<KIND>, dim3(kCUs), dim3(threads), 0, 0, src, out, clk, iters);
  };
  launch();  // warm-up, also brings the chip to its sustained clock
  if (hipDeviceSynchronize() != hipSuccess) return false;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return false;
  hipEventRecord(e0);
  launch();
  hipEventRecord(e1);
  if (hipEventSynchronize(e1) != hipSuccess) return false;
  float ms = 0.f;
  hipEventElapsedTime(&ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  std::vector<unsigned long long> c(4 * kCUs);
  if (hipMemcpy(c.data(), clk, c.size() * 8, hipMemcpyDeviceToHost) != hipSuccess) return false;
  double cyc = 0, real = 0;
  for (int g = 0; g < kCUs; ++g) {
    cyc += (double)(c[4 * g + 1] - c[4 * g]);
    real += (double)(c[4 * g + 3] - c[4 * g + 2]);
  }
  const double flops_per_mfma = KIND == 2 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
  const double flops = flops_per_mfma * 16.0 * iters * (4.0 * wps) * kCUs;
  r->ms = ms;
  r->tflops = flops / (ms * 1e-3) / 1e12;
  r->ghz = cyc / real * 0.1;  // s_memrealtime counts at 100 MHz
  return true;
}

int main() {
  uint32_t* src;
  float* out;
  unsigned long long* clk;
  CHECK(hipMalloc(&src, 4096 * 32 * sizeof(uint32_t)));
  CHECK(hipMalloc(&out, kCUs * 1024 * sizeof(float)));
  CHECK(hipMalloc(&clk, 4 * kCUs * sizeof(unsigned long long)));
  std::mt19937 rng(11);
  std::vector<uint32_t> h(4096 * 32);
  // Operand words: random signs and mantissas with magnitudes in [0.5, 2)
  // (bf16) or [0.5, 1) (fp16, e4m3), or the constant 1.0.
  auto fill = [&](int mode, int kind) {
    for (auto& x : h) {
      if (mode == 1) {  // constant 1.0 everywhere
        x = kind == 0 ? 0x3f803f80u : kind == 1 ? 0x3c003c00u : 0x38383838u;
        continue;
      }
      const uint32_t r = rng();
      if (kind == 0) x = (r & 0x807f807fu) | 0x3f003f00u | ((r >> 7) & 0x00800080u);
      else if (kind == 1) x = (r & 0x83ff83ffu) | 0x38003800u;
      else x = (r & 0x87878787u) | 0x30303030u;
    }
  };
  const char* kinds[3] = {"bf16 32x32x16", "fp16 32x32x16", "fp8 32x32x64 (scaled)"};
  const double peak[3] = {2516.6, 2516.6, 5033.2};
  std::printf("| MFMA | operands | waves per SIMD | TFLOP/s | %% of nominal peak | core clock (GHz) |\n");
  std::printf("|---|---|---|---|---|---|\n");
  for (int kind = 0; kind < 3; ++kind)
    for (int mode = 0; mode < 2; ++mode)
      for (int wps : {1, 2}) {
        fill(mode, kind);
        CHECK(hipMemcpy(src, h.data(), h.size() * sizeof(uint32_t), hipMemcpyHostToDevice));
        Run r;
        const int iters = kind == 2 ? 40000 / wps : 80000 / wps;  // about 20 ms
        bool ok = kind == 0   ? run<0>(src, out, clk, wps, iters, &r)
                  : kind == 1 ? run<1>(src, out, clk, wps, iters, &r)
                              : run<2>(src, out, clk, wps, iters, &r);
        if (!ok) {
          std::fprintf(stderr, "launch failed\n");
          return 1;
        }
        std::printf("| %s | %s | %d | %.0f | %.1f | %.2f |\n", kinds[kind],
                    mode ? "constant 1.0" : "random", wps, r.tflops, 100.0 * r.tflops / peak[kind],
                    r.ghz);
      }
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  return 0;
}

// dq_atomic_adds -- measures the dQ traffic that a dK/dV pass computing dQ by
// fp32 atomic adds would issue (the FLASH-ATTN page's FlashAttention-2
// "Parallelism" paragraph: the column-block workers of the backward
// communicate dQ through atomic adds), without any of that pass's other work.
//
// Workload: the d = 128 dK/dV grid at B1 H32 N16384 (non-causal): one
// workgroup of four waves per (head, key block of 128 keys), 4096 in all,
// each walking the 512 query tiles of 32 rows in order, as the dK/dV pass
// does.  Per tile a workgroup adds one 32 x 128 fp32 dQ tile: wave w adds the
// 32 columns 32 w .. 32 w + 31 from the MFMA C layout of dQ = dS K (lane
// (n, h), register r -> row 8 (r / 4) + 4 h + r % 4, column 32 w + n), i.e.
// 16 no-return global_atomic_add_f32 per lane, each wave instruction
// covering two full 128-byte lines.  Prints the time per launch and the rate.
//
// Build: hipcc --offload-arch=gfx950 -O3 -munsafe-fp-atomics
//        exact_attention_79_amd/probes/dq_atomic_adds.hip -o <exe>
// (build.py does this and places the program next to this file).
#include <hip/hip_runtime.h>

#include <cstdio>

#define CHECK(x)                                                      \
  do {                                                                \
    hipError_t e_ = (x);                                              \
    if (e_ != hipSuccess) {                                           \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));    \
      return 1;                                                       \
    }                                                                 \
  } while (0)

constexpr int kD = 128, kKeysPerBlock = 128, kTileRows = 32;

__global__ __launch_bounds__(256) void dq_atomic_adds(float* dq, int N, float v) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5;
  const int head = blockIdx.x / (N / kKeysPerBlock);
  float* base = dq + (size_t)head * N * kD;
  for (int t = 0; t < N / kTileRows; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = t * kTileRows + 8 * (r >> 2) + 4 * h + (r & 3);
      unsafeAtomicAdd(base + (size_t)row * kD + 32 * w + n, v);
    }
  }
}

int main() {
  const int H = 32, N = 16384, blocks = H * (N / kKeysPerBlock), reps = 3;
  const size_t elems = (size_t)H * N * kD;
  float* dq = nullptr;
  CHECK(hipMalloc(&dq, elems * sizeof(float)));
  CHECK(hipMemset(dq, 0, elems * sizeof(float)));
  hipLaunchKernelGGL(dq_atomic_adds, dim3(blocks), dim3(256), 0, 0, dq, N, 1.0f);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0));
  for (int i = 0; i < reps; ++i)
    hipLaunchKernelGGL(dq_atomic_adds, dim3(blocks), dim3(256), 0, 0, dq, N, 1.0f);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  ms /= reps;
  // Every workgroup of a head adds 1 to every element once per launch.
  float x = 0.f;
  CHECK(hipMemcpy(&x, dq, sizeof(float), hipMemcpyDeviceToHost));
  const double bytes = (double)blocks * (N / kTileRows) * kTileRows * kD * sizeof(float);
  std::printf("dQ by atomic adds, B1 H32 N16384 d128 dK/dV grid (%d workgroups): %.3f ms per "
              "launch, %.1f GB added, %.2f TB/s; check %s\n",
              blocks, ms, bytes / 1e9, bytes / (ms * 1e-3) / 1e12,
              x == (float)((reps + 1) * (N / kKeysPerBlock)) ? "ok" : "FAILED");
  CHECK(hipFree(dq));
  return x == (float)((reps + 1) * (N / kKeysPerBlock)) ? 0 : 1;
}

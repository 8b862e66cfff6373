// attn_kernels.hpp -- host-side launch interface between the C ABI layer and
// the HIP kernels (internal; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace attn {

// Dropout on P for the bf16 forward and backward (thresh = 0: none).
struct DropoutArgs {
  uint32_t thresh;     // bytes below it are dropped: round(256 p)
  uint32_t offset;     // fourth counter word
  uint64_t seed;       // Philox key
};

// BH = B * H query heads; K and V (and dK, dV) have B * Hkv heads, and query
// head h of batch b reads key/value head b * Hkv + h / (H / Hkv).
struct FwdArgs {
  const void* q;       // bf16 [BH][N][d], or e4m3 codes for the fp8 kernel
  const void* k;       // [B*Hkv][N][d]
  const void* v;
  void* o;             // bf16 or fp32 [BH][N][d]
  float* lse;          // fp32 [BH][N] or nullptr
  int BH, H, Hkv, N, d;
  float scale;         // softmax scale s
  int causal, window;
  int out_f32;         // 1: o is fp32, 0: bf16
  float q_descale, k_descale, v_descale;  // fp8 only: one per tensor, or
  const float* q_scales;  // ... one per block (nullptr: per tensor): [BH][N/128]
  const float* k_scales;  // [B*Hkv][N/64]
  const float* v_scales;  // [B*Hkv][N/64]
  DropoutArgs drop;    // bf16 kernel only
};

struct BwdArgs {
  const void* q;       // bf16 [BH][N][d]
  const void* k;       // bf16 [B*Hkv][N][d]
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;    // fp32 [BH][N]
  float* dq;           // fp32 [BH][N][d]
  float* dk;           // fp32 [B*Hkv][N][d], summed over each head group
  float* dv;
  float* delta;        // fp32 [BH][N] workspace: D_i = sum_k dO_ik O_ik
  float* lse2;         // fp32 [BH][N] workspace: L_i log2(e)
  float* dk_part;      // workspace, when dkdv_split > 1: fp32 [split][B*Hkv][N][d]
  float* dv_part;      //   partial dK, dV of each share of the query heads
  int BH, H, Hkv, N, d;
  float scale;
  int causal, window;
  DropoutArgs drop;
  int no_split;        // 1: the dK/dV pass never splits a group (no partials)
};

// A block of Nq queries (the last Nq positions) against Nk keys, split over
// the keys into P chunks whose partial results are merged.
struct DecodeArgs {
  const void* q;       // bf16 [B*H][Nq][d]
  const void* k;       // bf16 [B*Hkv][Nk][d]
  const void* v;
  void* o;             // bf16 or fp32 [B*H][Nq][d]
  float* lse;          // fp32 [B*H][Nq] or nullptr
  float* opart;        // workspace: fp32 [B*H*Nq][P][d]
  float* lpart;        // workspace: fp32 [B*H*Nq][P]
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  int causal, window, out_f32;
};
struct DecodePlan {
  int G, R, RB;        // query heads per key/value head, their rows, row blocks
  int P, CW, kmin;     // chunks, keys per chunk, first key any row sees
};
DecodePlan decode_plan(int B, int H, int Hkv, int Nq, int Nk, int window);

// The dK/dV pass gives each key block of a key/value head to one workgroup,
// which walks the query heads of its group (G = H / Hkv) and sums dK, dV over
// them in registers.  When that grid is too small for the chip (less than
// one round of workgroups over the 256 CUs, or, causal, less than two rounds,
// so that the uneven key blocks can even out), each group is split over
// `split` workgroups that write partial dK, dV to the workspace, summed by a
// second launch.  One round is 256 workgroups at d = 128 (one per CU) and
// 512 at d = 64 (two per CU).  Returns the smallest divisor of G that reaches
// the target, G if none does, 1 when there is nothing to split.
inline int dkdv_split(int BHkv, int G, int N, int d, int causal) {
  const long grid = (long)BHkv * ((N + 127) / 128);  // 128-key blocks
  const long want = 256L * (d == 64 ? 2 : 1) * (causal ? 2 : 1);
  if (G <= 1 || grid >= want) return 1;
  for (int s = 2; s < G; ++s)
    if (G % s == 0 && grid * s >= want) return s;
  return G;
}

// The symbol of a kernel instance as profilers list it, "attn::name<a, b>".
struct KName {
  const char* base;
  int n;
  int v[4];
  bool is_bool[4];
};
inline void kname_put(KName& k, int v) { k.is_bool[k.n] = false, k.v[k.n++] = v; }
inline void kname_put(KName& k, bool v) { k.is_bool[k.n] = true, k.v[k.n++] = v; }
template <typename... T>
inline KName kname(const char* base, T... t) {
  static_assert(sizeof...(T) <= 4, "at most four template arguments");
  KName k{base, 0, {}, {}};
  (kname_put(k, t), ...);
  return k;
}
inline std::string kname_str(const KName& k) {
  std::string s = k.base;
  s += '<';
  for (int i = 0; i < k.n; ++i) {
    if (i) s += ", ";
    s += k.is_bool[i] ? (k.v[i] ? "true" : "false") : std::to_string(k.v[i]);
  }
  return s + '>';
}

// Launches kernel K, or, when `name` is not null, launches nothing and
// returns the kernel's symbol there instead (static storage).  Each launch
// site states its kernel's template arguments once more in `sym`, on the
// same line as K.
template <auto K, typename... Args>
hipError_t go(const char** name, const KName& sym, dim3 grid, dim3 block, hipStream_t stream,
              Args... args) {
  if (name) {
    static const std::string s = kname_str(sym);
    *name = s.c_str();
    return hipSuccess;
  }
  hipLaunchKernelGGL(K, grid, block, 0, stream, args...);
  return hipGetLastError();
}

// Every launch function enqueues its kernels on `stream`; with `name` set it
// only reports the symbol of its main kernel (the one that does the
// attention arithmetic) for these arguments.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream, const char** name = nullptr);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// e4m3 inputs, widened in LDS, on the ping-pong forward (attn_fwd.hip).
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream, const char** name = nullptr);
// The backward stages; launch_bwd = dq (which also fills the workspace),
// then dkdv.  preprocess fills the workspace on its own.
hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream, const char** name = nullptr);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream, const char** name = nullptr);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace attn

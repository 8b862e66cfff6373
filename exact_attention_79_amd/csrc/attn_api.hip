// attn_api.hip -- the extern "C" boundary (include/attn.h): argument checks on
// the host, then one launch sequence on the caller's stream.  Nothing here
// allocates device memory or synchronises.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"
#include "attn_kernels.hpp"

// Device memory for callers that cannot allocate (attn_bwd_noalloc): the
// backward's D and L log2(e) arrays live here instead of in a caller's
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  Host code never uses the name `scratch` as an address (on
// the host it is only a stand-in for the symbol): the device address comes
// from hipGetSymbolAddress, once per device, in scratch_address below.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Key/value heads per batch element (H_kv = 0 means one per query head).
int kv_heads(const attn_desc* d) { return d->H_kv > 0 ? d->H_kv : d->H; }

attn_status check_desc(const attn_desc* d) {
  if (!d) return ATTN_EINVAL;
  if (d->B < 1 || d->H < 1 || d->N < 1) return ATTN_EINVAL;
  if (d->window < 0) return ATTN_EINVAL;
  if (d->causal != 0 && d->causal != 1) return ATTN_EINVAL;
  if (d->H_kv < 0 || (d->H_kv > 0 && d->H % d->H_kv != 0)) return ATTN_EINVAL;
  if (!isfinite(d->scale) || !(d->scale > 0.f)) return ATTN_EINVAL;
  if (d->d != 64 && d->d != 128) return ATTN_EUNSUPPORTED;
  const int64_t elems = (int64_t)d->B * d->H * d->N * d->d;
  if (elems >= ((int64_t)1 << 31)) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

attn_status check_ptrs(std::initializer_list<const void*> required,
                       std::initializer_list<const void*> optional) {
  for (const void* p : required)
    if (!p || !aligned16(p)) return ATTN_EINVAL;
  for (const void* p : optional)
    if (p && !aligned16(p)) return ATTN_EINVAL;
  return ATTN_OK;
}

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_EHIP; }

attn::FwdArgs fwd_args(const attn_desc* d, const void* q, const void* k,
                       const void* v, void* o, int32_t o_dtype, float* lse) {
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = d->B * d->H;
  a.H = d->H;
  a.Hkv = kv_heads(d);
  a.N = d->N;
  a.d = d->d;
  a.scale = d->scale;
  a.causal = d->causal;
  a.window = d->window;
  a.out_f32 = (o_dtype == ATTN_OUT_F32);
  a.q_descale = a.k_descale = a.v_descale = 1.f;
  a.q_scales = a.k_scales = a.v_scales = nullptr;
  a.drop = attn::DropoutArgs{0u, 0u, 0ull};
  return a;
}

// One fp32 [B,H,N] array of the workspace, padded to 256 bytes.
size_t ws_array_bytes(const attn_desc* d) {
  const size_t rows = (size_t)d->B * d->H * d->N;
  return (rows * sizeof(float) + 255) & ~(size_t)255;
}

// The partial dK (then dV) arrays of a split group walk, each padded to 256
// bytes; 0 when the dK/dV pass does not split (attn::dkdv_split).
size_t ws_share_bytes(const attn_desc* d) {
  const int split =
      attn::dkdv_split(d->B * kv_heads(d), d->H / kv_heads(d), d->N, d->d, d->causal);
  if (split <= 1) return 0;
  const size_t elems = (size_t)split * d->B * kv_heads(d) * d->N * d->d;
  return (elems * sizeof(float) + 255) & ~(size_t)255;
}

attn::BwdArgs bwd_args(const attn_desc* d, const void* q, const void* k,
                      const void* v, const void* o, const void* dout,
                      const float* lse, float* dq, float* dk, float* dv,
                      void* workspace) {
  attn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = (float*)workspace;
  a.lse2 = (float*)((char*)workspace + ws_array_bytes(d));
  a.dk_part = (float*)((char*)workspace + 2 * ws_array_bytes(d));
  a.dv_part = (float*)((char*)a.dk_part + ws_share_bytes(d));
  a.BH = d->B * d->H;
  a.H = d->H;
  a.Hkv = kv_heads(d);
  a.N = d->N;
  a.d = d->d;
  a.scale = d->scale;
  a.causal = d->causal;
  a.window = d->window;
  a.drop = attn::DropoutArgs{0u, 0u, 0ull};
  a.no_split = 0;
  return a;
}

// The keep threshold t = round(256 p) of a dropout description.
attn_status dropout_args(const attn_dropout* drop, attn::DropoutArgs* out) {
  if (!drop || !isfinite(drop->p) || drop->p < 0.f) return ATTN_EINVAL;
  const double t = floor((double)drop->p * 256.0 + 0.5);
  if (t > 255.0) return ATTN_EINVAL;
  out->thresh = (uint32_t)t;
  out->offset = drop->offset;
  out->seed = drop->seed;
  return ATTN_OK;
}

// The device address of `scratch` on the current device, looked up with that
// device current on the first call there and kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

attn_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_fwd(const attn_desc* desc, const void* q, const void* k,
                     const void* v, void* o, int32_t o_dtype, float* lse,
                     void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  if (o_dtype != ATTN_OUT_BF16 && o_dtype != ATTN_OUT_F32) return ATTN_EINVAL;
  st = check_ptrs({q, k, v, o}, {lse});
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_fwd_bf16(fwd_args(desc, q, k, v, o, o_dtype, lse),
                                        (hipStream_t)stream));
}

size_t attn_bwd_workspace_bytes(const attn_desc* desc) {
  if (check_desc(desc) != ATTN_OK) return 0;
  // D, then L log2(e), then the partial dK and dV of a split group walk.
  return 2 * ws_array_bytes(desc) + 2 * ws_share_bytes(desc);
}

attn_status attn_bwd(const attn_desc* desc, const void* q, const void* k,
                     const void* v, const void* o, const void* dout,
                     const float* lse, float* dq, float* dk, float* dv,
                     void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv, workspace}, {});
  if (st != ATTN_OK) return st;
  if (workspace_bytes < attn_bwd_workspace_bytes(desc)) return ATTN_EINVAL;
  return from_hip(attn::launch_bwd(
      bwd_args(desc, q, k, v, o, dout, lse, dq, dk, dv, workspace),
      (hipStream_t)stream));
}

size_t attn_bwd_noalloc_scratch_bytes(const attn_desc* desc) {
  if (check_desc(desc) != ATTN_OK) return 0;
  return 2 * ws_array_bytes(desc);
}

attn_status attn_bwd_noalloc(const attn_desc* desc, const void* q, const void* k,
                             const void* v, const void* o, const void* dout,
                             const float* lse, float* dq, float* dk, float* dv,
                             void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv}, {});
  if (st != ATTN_OK) return st;
  if (attn_bwd_noalloc_scratch_bytes(desc) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
    return ATTN_ESCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != ATTN_OK) return st;
  attn::BwdArgs a = bwd_args(desc, q, k, v, o, dout, lse, dq, dk, dv, ws);
  a.no_split = 1;  // no partial dK/dV arrays: the scratch holds D and L log2(e) only
  return from_hip(attn::launch_bwd(a, (hipStream_t)stream));
}

attn_status attn_bwd_preprocess(const attn_desc* desc, const void* o,
                                const void* dout, const float* lse, void* workspace,
                                size_t workspace_bytes, void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  st = check_ptrs({o, dout, lse, workspace}, {});
  if (st != ATTN_OK) return st;
  if (workspace_bytes < attn_bwd_workspace_bytes(desc)) return ATTN_EINVAL;
  return from_hip(attn::launch_bwd_preprocess(
      bwd_args(desc, nullptr, nullptr, nullptr, o, dout, lse, nullptr, nullptr,
               nullptr, workspace),
      (hipStream_t)stream));
}

attn_status attn_bwd_dq(const attn_desc* desc, const void* q, const void* k,
                        const void* v, const void* o, const void* dout,
                        const float* lse, void* workspace, size_t workspace_bytes,
                        float* dq, void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, o, dout, lse, workspace, dq}, {});
  if (st != ATTN_OK) return st;
  if (workspace_bytes < attn_bwd_workspace_bytes(desc)) return ATTN_EINVAL;
  return from_hip(attn::launch_bwd_dq(
      bwd_args(desc, q, k, v, o, dout, lse, dq, nullptr, nullptr, workspace),
      (hipStream_t)stream));
}

attn_status attn_bwd_dkdv(const attn_desc* desc, const void* q, const void* k,
                          const void* v, const void* dout, const void* workspace,
                          size_t workspace_bytes, float* dk, float* dv, void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, dout, workspace, dk, dv}, {});
  if (st != ATTN_OK) return st;
  if (workspace_bytes < attn_bwd_workspace_bytes(desc)) return ATTN_EINVAL;
  return from_hip(attn::launch_bwd_dkdv(
      bwd_args(desc, q, k, v, nullptr, dout, nullptr, nullptr, dk, dv,
               (void*)workspace),
      (hipStream_t)stream));
}

attn_status attn_fwd_dropout(const attn_desc* desc, const attn_dropout* drop,
                             const void* q, const void* k, const void* v, void* o,
                             int32_t o_dtype, float* lse, void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  if (o_dtype != ATTN_OUT_BF16 && o_dtype != ATTN_OUT_F32) return ATTN_EINVAL;
  st = check_ptrs({q, k, v, o}, {lse});
  if (st != ATTN_OK) return st;
  attn::FwdArgs a = fwd_args(desc, q, k, v, o, o_dtype, lse);
  st = dropout_args(drop, &a.drop);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_fwd_bf16(a, (hipStream_t)stream));
}

attn_status attn_bwd_dropout(const attn_desc* desc, const attn_dropout* drop,
                             const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, float* dq, float* dk,
                             float* dv, void* workspace, size_t workspace_bytes,
                             void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv, workspace}, {});
  if (st != ATTN_OK) return st;
  if (workspace_bytes < attn_bwd_workspace_bytes(desc)) return ATTN_EINVAL;
  attn::BwdArgs a = bwd_args(desc, q, k, v, o, dout, lse, dq, dk, dv, workspace);
  st = dropout_args(drop, &a.drop);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_bwd(a, (hipStream_t)stream));
}

attn_status attn_fwd_fp8(const attn_desc* desc, const uint8_t* q8,
                         const uint8_t* k8, const uint8_t* v8, float q_descale,
                         float k_descale, float v_descale, void* o,
                         int32_t o_dtype, float* lse, void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  if (o_dtype != ATTN_OUT_BF16 && o_dtype != ATTN_OUT_F32) return ATTN_EINVAL;
  for (float s : {q_descale, k_descale, v_descale})
    if (!isfinite(s) || !(s > 0.f)) return ATTN_EINVAL;
  st = check_ptrs({q8, k8, v8, o}, {lse});
  if (st != ATTN_OK) return st;
  attn::FwdArgs a = fwd_args(desc, q8, k8, v8, o, o_dtype, lse);
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  return from_hip(attn::launch_fwd_fp8(a, (hipStream_t)stream));
}

attn_status attn_fwd_fp8_blocks(const attn_desc* desc, const uint8_t* q8,
                                const uint8_t* k8, const uint8_t* v8,
                                const float* q_descales, const float* k_descales,
                                const float* v_descales, void* o, int32_t o_dtype,
                                float* lse, void* stream) {
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  if (o_dtype != ATTN_OUT_BF16 && o_dtype != ATTN_OUT_F32) return ATTN_EINVAL;
  st = check_ptrs({q8, k8, v8, o}, {lse});
  if (st != ATTN_OK) return st;
  if (!q_descales || !k_descales || !v_descales || ((uintptr_t)q_descales & 3) ||
      ((uintptr_t)k_descales & 3) || ((uintptr_t)v_descales & 3))
    return ATTN_EINVAL;
  attn::FwdArgs a = fwd_args(desc, q8, k8, v8, o, o_dtype, lse);
  a.q_scales = q_descales;
  a.k_scales = k_descales;
  a.v_scales = v_descales;
  return from_hip(attn::launch_fwd_fp8(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

attn_status check_decode_desc(const attn_decode_desc* d) {
  if (!d) return ATTN_EINVAL;
  if (d->B < 1 || d->H < 1 || d->N_q < 1 || d->N_k < 1 || d->N_q > d->N_k)
    return ATTN_EINVAL;
  if (d->window < 0 || (d->causal != 0 && d->causal != 1)) return ATTN_EINVAL;
  if (d->H_kv < 0 || (d->H_kv > 0 && d->H % d->H_kv != 0)) return ATTN_EINVAL;
  if (!isfinite(d->scale) || !(d->scale > 0.f)) return ATTN_EINVAL;
  if (d->d != 64 && d->d != 128) return ATTN_EUNSUPPORTED;
  const int64_t hkv = d->H_kv > 0 ? d->H_kv : d->H;
  if ((int64_t)d->B * d->H * d->N_q * d->d >= ((int64_t)1 << 31) ||
      (int64_t)d->B * hkv * d->N_k * d->d >= ((int64_t)1 << 31))
    return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

attn::DecodePlan decode_plan_of(const attn_decode_desc* d) {
  return attn::decode_plan(d->B, d->H, d->H_kv > 0 ? d->H_kv : d->H, d->N_q, d->N_k,
                           d->window);
}

size_t pad256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

size_t attn_decode_workspace_bytes(const attn_decode_desc* desc) {
  if (check_decode_desc(desc) != ATTN_OK) return 0;
  const attn::DecodePlan pl = decode_plan_of(desc);
  const size_t rows = (size_t)desc->B * desc->H * desc->N_q;
  return pad256(rows * pl.P * desc->d * sizeof(float)) + pad256(rows * pl.P * sizeof(float));
}

attn_status attn_fwd_decode(const attn_decode_desc* desc, const void* q, const void* k,
                            const void* v, void* o, int32_t o_dtype, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  attn_status st = check_decode_desc(desc);
  if (st != ATTN_OK) return st;
  if (o_dtype != ATTN_OUT_BF16 && o_dtype != ATTN_OUT_F32) return ATTN_EINVAL;
  st = check_ptrs({q, k, v, o, workspace}, {lse});
  if (st != ATTN_OK) return st;
  if (workspace_bytes < attn_decode_workspace_bytes(desc)) return ATTN_EINVAL;
  const attn::DecodePlan pl = decode_plan_of(desc);
  attn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.opart = (float*)workspace;
  a.lpart = (float*)((char*)workspace +
                     pad256((size_t)desc->B * desc->H * desc->N_q * pl.P * desc->d * 4));
  a.B = desc->B;
  a.H = desc->H;
  a.Hkv = desc->H_kv > 0 ? desc->H_kv : desc->H;
  a.Nq = desc->N_q;
  a.Nk = desc->N_k;
  a.d = desc->d;
  a.scale = desc->scale;
  a.causal = desc->causal;
  a.window = desc->window;
  a.out_f32 = (o_dtype == ATTN_OUT_F32);
  return from_hip(attn::launch_decode(a, (hipStream_t)stream));
}

const char* attn_kernel_name(const attn_desc* desc, int32_t stage, float dropout_p) {
  if (check_desc(desc) != ATTN_OK) return nullptr;
  attn::DropoutArgs drop{0u, 0u, 0ull};
  if (dropout_p != 0.f) {
    const attn_dropout dd{dropout_p, 0u, 0ull};
    if (dropout_args(&dd, &drop) != ATTN_OK || stage == ATTN_STAGE_FWD_FP8) return nullptr;
  }
  // Any aligned non-null stand-in: nothing is launched or dereferenced.
  void* x = (void*)(uintptr_t)256;
  const char* name = nullptr;
  hipError_t e = hipErrorInvalidValue;
  if (stage == ATTN_STAGE_FWD || stage == ATTN_STAGE_FWD_FP8) {
    attn::FwdArgs a = fwd_args(desc, x, x, x, x, ATTN_OUT_BF16, nullptr);
    a.drop = drop;
    e = stage == ATTN_STAGE_FWD ? attn::launch_fwd_bf16(a, nullptr, &name)
                                : attn::launch_fwd_fp8(a, nullptr, &name);
  } else if (stage == ATTN_STAGE_BWD_DQ || stage == ATTN_STAGE_BWD_DKDV) {
    attn::BwdArgs a = bwd_args(desc, x, x, x, x, x, (const float*)x, (float*)x, (float*)x,
                               (float*)x, x);
    a.drop = drop;
    e = stage == ATTN_STAGE_BWD_DQ ? attn::launch_bwd_dq(a, nullptr, &name)
                                   : attn::launch_bwd_dkdv(a, nullptr, &name);
  }
  return e == hipSuccess ? name : nullptr;
}

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK:
      return "ok";
    case ATTN_EINVAL:
      return "invalid argument";
    case ATTN_EUNSUPPORTED:
      return "unsupported shape (head dim must be 64 or 128; B*H*N*d < 2^31)";
    case ATTN_EHIP:
      return "HIP runtime error at launch";
    case ATTN_ESCRATCH:
      return "problem too large for the no-allocation entry point's static scratch "
             "(B*H*N above its limit)";
  }
  return "unknown status";
}

}  // extern "C"

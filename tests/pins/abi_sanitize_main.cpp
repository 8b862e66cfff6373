// Drives the host side of the C ABI (include/attn.h) through every check
// that happens before a launch -- descriptor, pointer, dtype, workspace and
// scratch validation, workspace sizes, kernel names, status strings -- for a
// build of the ABI layer under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Nothing here launches a kernel or touches a
// device, so it runs without a GPU.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    printf("%s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  char buf[64];
  void* F = (void*)(uintptr_t)0x10000;  // aligned, never dereferenced
  attn_desc ok = {2, 4, 100, 128, 0.125f, 1, 0, 0};
  // Descriptor checks of every entry point.
  attn_desc bad[] = {
      {0, 4, 100, 128, 0.125f, 1, 0, 0},     {2, 0, 100, 128, 0.125f, 1, 0, 0},
      {2, 4, 0, 128, 0.125f, 1, 0, 0},       {2, 4, 100, 128, 0.125f, 2, 0, 0},
      {2, 4, 100, 128, 0.125f, 1, -1, 0},    {2, 4, 100, 128, 0.f, 1, 0, 0},
      {2, 4, 100, 128, NAN, 1, 0, 0},        {2, 4, 100, 128, INFINITY, 1, 0, 0},
      {2, 4, 100, 128, 0.125f, 1, 0, 3},     {2, 4, 100, 128, 0.125f, 1, 0, -1}};
  for (const attn_desc& d : bad) {
    expect(attn_fwd(&d, F, F, F, F, ATTN_OUT_BF16, nullptr, nullptr), ATTN_EINVAL, "fwd desc");
    expect((int)attn_bwd_workspace_bytes(&d), 0, "bwd workspace of a bad desc");
    expect(attn_bwd(&d, F, F, F, F, F, (const float*)F, (float*)F, (float*)F, (float*)F, F,
                    1 << 20, nullptr),
           ATTN_EINVAL, "bwd desc");
    expect(attn_bwd_noalloc(&d, F, F, F, F, F, (const float*)F, (float*)F, (float*)F,
                            (float*)F, nullptr),
           ATTN_EINVAL, "noalloc desc");
    expect(attn_kernel_name(&d, ATTN_STAGE_FWD, 0.f) == nullptr, 1, "kernel name of a bad desc");
  }
  attn_desc d96 = ok;
  d96.d = 96;
  expect(attn_fwd(&d96, F, F, F, F, ATTN_OUT_BF16, nullptr, nullptr), ATTN_EUNSUPPORTED, "d 96");
  attn_desc huge = {1024, 1024, 1024, 128, 0.1f, 0, 0, 0};
  expect(attn_fwd(&huge, F, F, F, F, ATTN_OUT_BF16, nullptr, nullptr), ATTN_EUNSUPPORTED,
         "2^31 elements");
  expect(attn_fwd(nullptr, F, F, F, F, 0, nullptr, nullptr), ATTN_EINVAL, "null desc");
  // Pointer and dtype checks.
  expect(attn_fwd(&ok, nullptr, F, F, F, 0, nullptr, nullptr), ATTN_EINVAL, "null q");
  expect(attn_fwd(&ok, F, (char*)F + 8, F, F, 0, nullptr, nullptr), ATTN_EINVAL, "unaligned k");
  expect(attn_fwd(&ok, F, F, F, F, 7, nullptr, nullptr), ATTN_EINVAL, "o dtype");
  expect(attn_fwd(&ok, F, F, F, F, 0, (float*)((char*)F + 4), nullptr), ATTN_EINVAL, "lse");
  // Workspace sizes and the backward's workspace check.
  const size_t ws = attn_bwd_workspace_bytes(&ok);
  expect(ws >= 2 * 2 * 4 * 100 * 4 && ws % 256 == 0, 1, "workspace size");
  expect(attn_bwd(&ok, F, F, F, F, F, (const float*)F, (float*)F, (float*)F, (float*)F, F,
                  ws - 1, nullptr),
         ATTN_EINVAL, "small workspace");
  expect(attn_bwd_dq(&ok, F, F, F, F, F, (const float*)F, F, ws - 1, (float*)F, nullptr),
         ATTN_EINVAL, "dq workspace");
  expect(attn_bwd_dkdv(&ok, F, F, F, F, F, ws, (float*)F, nullptr, nullptr), ATTN_EINVAL,
         "dkdv null dv");
  expect(attn_bwd_preprocess(&ok, F, F, nullptr, F, ws, nullptr), ATTN_EINVAL, "preprocess lse");
  attn_desc gqa = {4, 16, 2048, 64, 0.125f, 1, 0, 4};
  expect(attn_bwd_workspace_bytes(&gqa) > 2 * (size_t)4 * 16 * 2048 * 4, 1, "split partials");
  // The no-allocation backward's scratch limit.
  attn_desc big = {1, 64, 65536, 64, 0.1f, 1, 0, 0};
  expect(attn_bwd_noalloc_scratch_bytes(&big) > ATTN_NOALLOC_SCRATCH_BYTES, 1, "scratch need");
  expect(attn_bwd_noalloc(&big, F, F, F, F, F, (const float*)F, (float*)F, (float*)F, (float*)F,
                          nullptr),
         ATTN_ESCRATCH, "noalloc over the scratch");
  // fp8 descales and block descales.
  expect(attn_fwd_fp8(&ok, (const uint8_t*)F, (const uint8_t*)F, (const uint8_t*)F, 0.f, 1.f, 1.f,
                      F, 0, nullptr, nullptr),
         ATTN_EINVAL, "fp8 descale");
  expect(attn_fwd_fp8_blocks(&ok, (const uint8_t*)F, (const uint8_t*)F, (const uint8_t*)F,
                             nullptr, (const float*)F, (const float*)F, F, 0, nullptr, nullptr),
         ATTN_EINVAL, "fp8 block descales");
  // Dropout descriptions.
  attn_dropout dr = {0.999f, 0, 1};
  expect(attn_fwd_dropout(&ok, &dr, F, F, F, F, 0, nullptr, nullptr), ATTN_EINVAL, "dropout p");
  expect(attn_fwd_dropout(&ok, nullptr, F, F, F, F, 0, nullptr, nullptr), ATTN_EINVAL,
         "null dropout");
  // Decode.
  attn_decode_desc dd = {2, 8, 2, 1, 5000, 128, 0.1f, 0, 0};
  const size_t dws = attn_decode_workspace_bytes(&dd);
  expect(dws > 0 && dws % 256 == 0, 1, "decode workspace");
  expect(attn_fwd_decode(&dd, F, F, F, F, 0, nullptr, F, dws - 1, nullptr), ATTN_EINVAL,
         "decode workspace check");
  dd.N_q = 6000;
  expect((int)attn_decode_workspace_bytes(&dd), 0, "decode N_q > N_k");
  // Kernel names and status strings.
  const char* n1 = attn_kernel_name(&ok, ATTN_STAGE_FWD, 0.f);
  const char* n2 = attn_kernel_name(&ok, ATTN_STAGE_BWD_DKDV, 0.1f);
  expect(n1 && n2 && strncmp(n1, "attn::", 6) == 0 && strncmp(n2, "attn::", 6) == 0, 1, "names");
  expect(attn_kernel_name(&ok, 9, 0.f) == nullptr, 1, "bad stage");
  expect(attn_kernel_name(&ok, ATTN_STAGE_FWD_FP8, 0.1f) == nullptr, 1, "fp8 dropout");
  for (int s = 0; s <= 5; ++s) snprintf(buf, sizeof buf, "%s", attn_status_str((attn_status)s));
  printf("ABI layer under sanitizers: %s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}

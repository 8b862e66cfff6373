"""Register and scratch use of the compiled kernels (CPU only: hipcc
cross-compiles the device code for gfx950 and reports each kernel's
resources).

A kernel whose register arrays are indexed with values the compiler cannot
fold (a loop it did not unroll), or whose live registers exceed the budget
of its waves per SIMD, runs from scratch memory, many times slower and with
the same results; no parity test notices.  The hot-path kernels must use
no scratch and spill no vector register; the others (dropout, d = 64 single
wave) are held to the few spilled registers they have now.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "exact_attention_79_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Kernels (by mangled-name fragment) that must use no scratch and spill no
# vector register.
HOT = ["fwd_pp_kernel", "fwd_fp8_pp_kernel", "bwd_dq_pp_kernel", "bwd_dkdv_quad_kernel",
       "bwd_dkdv_pp_kernel", "bwd_delta_kernel", "decode_split_kernel", "decode_merge_kernel"]
# Bytes of scratch per lane allowed to the other kernels.
OTHER_MAX_SCRATCH = 64


def _resources(src, tmp_path):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "--cuda-device-only", "-c",
           os.path.join(CSRC, src), "-o", str(tmp_path / (src + ".o")),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark: ([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", ["attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip"])
def test_no_scratch_in_hot_kernels(src, tmp_path):
    kernels = _resources(src, tmp_path)
    assert kernels, "no kernel resource remarks parsed"
    for name, res in kernels.items():
        assert "ScratchSize" in res and "VGPRs Spill" in res, (name, res)
        if any(h in name for h in HOT):
            assert res["ScratchSize"] == 0 and res["VGPRs Spill"] == 0, (name, res)
        else:
            assert res["ScratchSize"] <= OTHER_MAX_SCRATCH, (name, res)

"""The largest problem the library accepts: B*H*N*d just under 2^31 elements
(B1 H8191 N2048 d128, 4.3 GB per bf16 tensor), forward and backward, the fp8
forward at that size, and the rejection one head above it.

Heads are independent, so only the checked heads need oracle inputs: the
first, a middle and the last head get the seeded host-generated bf16 values
(the same generator as every other test), the rest are filled on the device
with torch's seeded generator.  The checked heads are compared in full
against the oracle at the usual bars (O, dQ, dK, dV max abs <= 2e-2, mean abs
<= 2e-3; LSE max abs <= 1e-3); the offsets of the last head exercise the
largest byte offsets the kernels form.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import BF16_MAX, BF16_MEAN, LSE_MAX, assert_close, bf16_case, log

pytestmark = pytest.mark.gpu

B, H, N, D = 1, 8191, 2048, 128
CHECKED = (0, 4095, H - 1)


@pytest.fixture(scope="module")
def ea():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import exact_attention_79_amd as ea
    return ea


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def big(ea):
    assert B * H * N * D < 2 ** 31 <= B * (H + 1) * N * D
    log(f"case: limits B{B} H{H} N{N} d{D} ({B * H * N * D} elements per tensor)")
    gen = torch.Generator(device="cuda").manual_seed(31)
    t = {n: torch.randn((B, H, N, D), device="cuda", generator=gen).bfloat16()
         for n in ("q", "k", "v", "do")}
    ref = {}
    for i, h in enumerate(CHECKED):
        dev, r = bf16_case(3100 + i, 1, 1, N, D, with_dout=True)
        for n in ("q", "k", "v", "do"):
            t[n][0, h].copy_(dev[n][0, 0])
        ref[h] = r
    torch.cuda.synchronize()
    yield t, ref
    del t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_largest_forward_and_backward(ea, big, causal):
    t, ref = big
    s = 1 / math.sqrt(D)
    o, lse = ea.attn_fwd(t["q"], t["k"], t["v"], causal=causal)
    dq, dk, dv = ea.attn_bwd(t["q"], t["k"], t["v"], o, t["do"], lse, causal=causal)
    torch.cuda.synchronize()
    for h in CHECKED:
        r = ref[h]
        o_r, l_r = oracle.fwd(r["q"], r["k"], r["v"], s, causal)
        assert_close(np64(o[0, h]), o_r[0, 0], BF16_MAX, BF16_MEAN, f"O head {h}")
        assert_close(np64(lse[0, h]), l_r[0, 0], LSE_MAX, None, f"LSE head {h}")
        want = oracle.bwd(r["q"], r["k"], r["v"], r["do"], s, causal)[:3]
        for name, g, w in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
            assert_close(np64(g[0, h]), w[0, 0], BF16_MAX, BF16_MEAN, f"{name} head {h}")
    del o, lse, dq, dk, dv


@pytest.mark.parametrize("causal", [False, True])
def test_largest_fp8_forward(ea, causal):
    """The fp8 forward at the same size (e4m3 codes, 2.1 GB per tensor):
    the checked heads carry the fp8 workload recipe's codes (one x10 outlier
    channel) and the tensors' descales; the other heads are device-drawn
    codes under the same descales."""
    import attn_synth
    from helpers import FP8_MAX
    gen = torch.Generator(device="cuda").manual_seed(32)
    t = {}
    for n in ("q", "k", "v"):
        t[n] = torch.empty((B, H, N, D), device="cuda", dtype=torch.uint8)
        for h0 in range(0, H, 1024):
            x = torch.randn((B, min(1024, H - h0), N, D), device="cuda", generator=gen)
            t[n][:, h0:h0 + x.shape[1]] = (x * 16).to(torch.float8_e4m3fn).view(torch.uint8)
            del x
    f8 = attn_synth.fp8_attention_inputs(3200, 1, len(CHECKED), N, D)
    for i, h in enumerate(CHECKED):
        for n in ("q", "k", "v"):
            t[n][0, h].copy_(torch.from_numpy(f8[n][0, i]))
    s = 1 / math.sqrt(D)
    o, lse = ea.attn_fwd_fp8(t["q"], t["k"], t["v"], f8["q_descale"], f8["k_descale"],
                             f8["v_descale"], causal=causal)
    torch.cuda.synchronize()
    ref = {n: oracle.decode_e4m3(f8[n], f8[n + "_descale"]) for n in ("q", "k", "v")}
    for i, h in enumerate(CHECKED):
        o_r, _ = oracle.fwd(ref["q"][0, i], ref["k"][0, i], ref["v"][0, i], s, causal)
        assert_close(np64(o[0, h]), o_r, FP8_MAX, None, f"fp8 O head {h}")
    del o, lse, t
    torch.cuda.empty_cache()


def test_one_head_more_is_refused(ea):
    import ctypes
    desc = ea.make_desc(B, H + 1, N, D, 1 / math.sqrt(D), False, 0)
    vp = ctypes.c_void_p
    f = vp(0x10000)
    assert ea.lib.attn_fwd(ctypes.byref(desc), f, f, f, f, 0, None, None) == \
        ea.ATTN_EUNSUPPORTED
    assert ea.lib.attn_bwd_workspace_bytes(ctypes.byref(desc)) == 0

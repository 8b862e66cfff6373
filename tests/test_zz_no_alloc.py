"""The no-allocation backward (attn_bwd_noalloc, for callers that cannot
allocate) through the C ABI against the ordinary backward (attn_bwd with a
caller workspace) on the same inputs: two calls in a row, the second on a
smaller problem, so the second runs on scratch the first left behind; and a
grouped-query case that attn_bwd splits (partial dK/dV in its workspace)
while the no-allocation path walks whole groups.

Bar: the ordinary backward's outputs, max abs <= 2e-2 and mean abs <= 2e-3
(the bf16 gradient bar); where the two run the same kernels the outputs must
also be bitwise equal.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

from helpers import BF16_MAX, BF16_MEAN, assert_close, bf16_case, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import exact_attention_79_amd as ea
    return ea


def guarded(shape):
    """An fp32 output carved out of a buffer whose margins hold a sentinel."""
    n, pad = int(np.prod(shape)), 64
    buf = torch.full((n + 2 * pad,), 7.0, device="cuda")
    return buf, buf[pad:pad + n].view(shape)


def margins_intact(buf):
    return bool((buf[:64] == 7.0).all()) and bool((buf[-64:] == 7.0).all())


def noalloc_through_abi(ea, q, k, v, o, do, lse, causal, window):
    bufs, grads = zip(*(guarded(q.shape), guarded(k.shape), guarded(k.shape)))
    B, H, N, d = q.shape
    desc = ea.make_desc(B, H, N, d, 1 / math.sqrt(d), causal, window, k.shape[1])
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ea.lib.attn_bwd_noalloc(ctypes.byref(desc), p(q), p(k), p(v), p(o), p(do), p(lse),
                                 *(p(g) for g in grads),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ea.ATTN_OK, ea.status_str(st)
    torch.cuda.synchronize()
    assert all(margins_intact(b) for b in bufs), "kernel wrote outside its outputs"
    return grads


def compare(ea, workload, B, H, Hkv, N, d, causal, window, bitwise):
    log(f"case: no-alloc bwd B{B} H{H} H_kv{Hkv} N{N} d{d} causal={causal} window={window}")
    dev, _ = bf16_case(workload, B, H, N, d, with_dout=True)
    q, do = dev["q"], dev["do"]
    k, v = dev["k"][:, :Hkv].contiguous(), dev["v"][:, :Hkv].contiguous()
    o, lse = ea.attn_fwd(q, k, v, causal=causal, window=window)
    want = ea.attn_bwd(q, k, v, o, do, lse, causal=causal, window=window)
    got = noalloc_through_abi(ea, q, k, v, o, do, lse, causal, window)
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        assert_close(g.cpu().numpy(), w.cpu().numpy().astype(np.float64), BF16_MAX, BF16_MEAN,
                     f"{name} vs attn_bwd")
        if bitwise:
            assert torch.equal(g, w), f"{name}: not bitwise equal to attn_bwd"


def test_two_calls_second_smaller(ea):
    compare(ea, 810, 2, 4, 4, 1000, 128, True, 0, bitwise=True)
    compare(ea, 811, 1, 2, 2, 300, 64, False, 65, bitwise=True)


def test_grouped_query_without_split(ea):
    """attn_bwd splits this group walk over 8 workgroups (partials summed by a
    second launch); the no-allocation path walks whole groups."""
    assert ea.attn_bwd_workspace_bytes(1, 8, 2048, 64, 1, False) > 2 * 8 * 2048 * 4
    compare(ea, 812, 1, 8, 1, 2048, 64, False, 0, bitwise=False)


def test_rejects_problems_beyond_the_scratch(ea):
    q = torch.empty((1, 64, 65536, 64), device="cuda", dtype=torch.bfloat16)
    grads = (torch.empty(q.shape, device="cuda", dtype=torch.float32),) * 3
    lse = torch.empty((1, 64, 65536), device="cuda", dtype=torch.float32)
    with pytest.raises(ea.AttnError) as err:
        ea.attn_bwd_noalloc(q, q, q, q, q, lse, grads)
    assert err.value.status == ea.ATTN_ESCRATCH

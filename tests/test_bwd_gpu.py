"""Parity of the bf16 backward (through the C ABI) against the fp64 oracle.

The forward's own bf16 O and fp32 LSE feed the backward, as in training; the
oracle's gradients are exact functions of the same bf16 inputs.
Bars: dQ, dK, dV max abs <= 2e-2 and mean abs <= 2e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import BF16_MAX, BF16_MEAN, assert_close, bf16_case, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import exact_attention_79_amd as ea
    return ea


def fwd_bwd(ea, dev, causal, window):
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = ea.attn_fwd(q, k, v, causal=causal, window=window)
    B, H, N, d = q.shape
    pad = 64
    bufs = [torch.full((q.numel() + 2 * pad,), 7.0, device="cuda") for _ in range(3)]
    grads = tuple(b[pad:pad + q.numel()].view(q.shape) for b in bufs)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, do, lse, causal=causal, window=window,
                             grads=grads)
    torch.cuda.synchronize()
    for b in bufs:
        assert (b[:pad] == 7.0).all() and (b[-pad:] == 7.0).all(), \
            "kernel wrote outside its outputs"
    return [t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]


SMALL = [(1, 64), (17, 128), (100, 64), (257, 128), (333, 64), (520, 128)]
MASKS = [(False, 0), (True, 0), (True, 1), (True, 65), (False, 40), (True, 10**6)]


@pytest.mark.parametrize("N,d", SMALL)
@pytest.mark.parametrize("causal,window", MASKS)
def test_ragged_shapes_and_masks(ea, N, d, causal, window):
    log(f"case: bwd B2 H2 N{N} d{d} causal={causal} window={window}")
    dev, ref = bf16_case(400 + N, 2, 2, N, d, with_dout=True)
    got = fwd_bwd(ea, dev, causal, window)
    want = oracle.bwd(ref["q"], ref["k"], ref["v"], ref["do"], 1 / math.sqrt(d),
                      causal, window)[:3]
    for name, g, r in zip(("dQ", "dK", "dV"), got, want):
        assert_close(g, r, BF16_MAX, BF16_MEAN, name)


def test_backward_full_size_two_heads(ea):
    """B=4, H=16, N=4096, d=128 causal; heads (0,0) and (3,15) compared in full."""
    B, H, N, d = 4, 16, 4096, 128
    log(f"case: bwd B{B} H{H} N{N} d{d} causal")
    dev, ref = bf16_case(4, B, H, N, d, with_dout=True)
    got = fwd_bwd(ea, dev, True, 0)
    for b, h in ((0, 0), (B - 1, H - 1)):
        want = oracle.bwd(ref["q"][b, h], ref["k"][b, h], ref["v"][b, h],
                          ref["do"][b, h], 1 / math.sqrt(d), True, 0)[:3]
        for name, g, r in zip(("dQ", "dK", "dV"), got, want):
            assert_close(g[b, h], r, BF16_MAX, BF16_MEAN, f"{name} head ({b},{h})")
    for g in got:
        assert np.isfinite(g).all()


@pytest.mark.parametrize("d", [64, 128])
def test_gradient_invariants(ea, d):
    """sum_j dK_j = 0 (rows of dS sum to zero); constant V gives dQ = dK = 0."""
    N = 700
    log(f"case: bwd invariants N{N} d{d}")
    dev, _ = bf16_case(500 + d, 1, 2, N, d, with_dout=True)
    dq, dk, dv = fwd_bwd(ea, dev, True, 0)
    log(f"    max |sum_j dK_j| = {np.abs(dk.sum(axis=2)).max():.3e}")
    assert np.abs(dk.sum(axis=2)).max() < 5e-2
    dev["v"] = dev["v"][:, :, :1, :].expand(-1, -1, N, -1).contiguous()
    dq, dk, dv = fwd_bwd(ea, dev, True, 0)
    assert np.abs(dq).max() < 2e-2 and np.abs(dk).max() < 2e-2


def test_backward_deterministic(ea):
    log("case: bwd determinism B2 H3 N999 d128 causal")
    dev, _ = bf16_case(600, 2, 3, 999, 128, with_dout=True)
    a = fwd_bwd(ea, dev, True, 0)
    b = fwd_bwd(ea, dev, True, 0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)

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
from helpers import BF16_MAX, BF16_MEAN, LSE_MAX, assert_close, bf16_case, log

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


# At d = 128 the dK/dV pass walks 32-row query tiles in a loop unrolled six
# steps deep: U tiles take U + 3 steps, its four wave roles running up to
# three tiles apart.  Non-causal, every key block walks N / 32 tiles: N = 32
# .. 384 covers walks of 1 to 12 tiles (every remainder of the unrolled loop,
# twice); causal at N = 416 the four key blocks walk 13, 9, 5 and 1.
@pytest.mark.parametrize("N,causal", [(32 * u, False) for u in range(1, 13)] + [(416, True)])
def test_dkdv_tile_walk_lengths(ea, N, causal):
    d = 128
    log(f"case: bwd B1 H2 N{N} d{d} causal={causal} (dK/dV walk lengths)")
    dev, ref = bf16_case(470 + N, 1, 2, N, d, with_dout=True)
    got = fwd_bwd(ea, dev, causal, 0)
    want = oracle.bwd(ref["q"], ref["k"], ref["v"], ref["do"], 1 / math.sqrt(d), causal, 0)[:3]
    for name, g, r in zip(("dQ", "dK", "dV"), got, want):
        assert_close(g, r, BF16_MAX, BF16_MEAN, name)


# At d = 64 the forward walks 64-key tiles (a loop unrolled three steps deep)
# and the non-causal dK/dV pass 32-row query tiles (four deep): N = 64 .. 512
# covers walks of 1 to 8 and 2 to 16 tiles; causal at N = 576 exercises the
# forward's first group stopping early.
@pytest.mark.parametrize("N,causal", [(64 * u, False) for u in range(1, 9)] + [(576, True)])
def test_d64_tile_walk_lengths(ea, N, causal):
    d = 64
    log(f"case: bwd B1 H2 N{N} d{d} causal={causal} (d = 64 walk lengths)")
    dev, ref = bf16_case(490 + N, 1, 2, N, d, with_dout=True)
    o, lse = ea.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    o_ref, lse_ref = oracle.fwd(ref["q"], ref["k"], ref["v"], 1 / math.sqrt(d), causal)
    assert_close(o.float().cpu().numpy().astype(np.float64), o_ref, BF16_MAX, BF16_MEAN, "O")
    assert_close(lse.cpu().numpy().astype(np.float64), lse_ref, LSE_MAX, None, "LSE")
    got = fwd_bwd(ea, dev, causal, 0)
    want = oracle.bwd(ref["q"], ref["k"], ref["v"], ref["do"], 1 / math.sqrt(d), causal, 0)[:3]
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
@pytest.mark.parametrize("causal", [False, True])
def test_backward_step_shape_two_heads(ea, d, causal):
    """The backward launches bench.py times: B=4, H=16, N=2048, d in {64, 128},
    causal and non-causal; heads (0,0) and (3,15) compared in full."""
    B, H, N = 4, 16, 2048
    log(f"case: bwd B{B} H{H} N{N} d{d} causal={causal}")
    dev, ref = bf16_case(2, B, H, N, d, with_dout=True)
    got = fwd_bwd(ea, dev, causal, 0)
    for b, h in ((0, 0), (B - 1, H - 1)):
        want = oracle.bwd(ref["q"][b, h], ref["k"][b, h], ref["v"][b, h],
                          ref["do"][b, h], 1 / math.sqrt(d), causal, 0)[:3]
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


@pytest.mark.parametrize("d,causal", [(64, False), (128, True)])
def test_stages_and_workspace(ea, d, causal):
    """attn_bwd_stages (dQ pass, then dK/dV pass) is bitwise attn_bwd; the
    preprocess-filled workspace (D, L log2 e) agrees with the one the dQ pass
    writes, and dK, dV computed from it meet the bars against the oracle."""
    B, H, N = 2, 2, 777
    log(f"case: bwd stages B{B} H{H} N{N} d{d} causal={causal}")
    dev, ref = bf16_case(700 + d, B, H, N, d, with_dout=True)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = ea.attn_fwd(q, k, v, causal=causal)
    whole = ea.attn_bwd(q, k, v, o, do, lse, causal=causal)
    nbytes = ea.attn_bwd_workspace_bytes(B, H, N, d)
    ws_dq = torch.zeros(nbytes, device="cuda", dtype=torch.uint8)
    staged = ea.attn_bwd_stages(q, k, v, o, do, lse, causal=causal, workspace=ws_dq)
    ws_pre = torch.zeros(nbytes, device="cuda", dtype=torch.uint8)
    pre = ea.attn_bwd_stages(q, k, v, o, do, lse, causal=causal, workspace=ws_pre,
                             preprocess=True)
    # the preprocess pass alone, on a fresh workspace
    ws_only = torch.zeros(nbytes, device="cuda", dtype=torch.uint8)
    ea.attn_bwd_preprocess(o, do, lse, ws_only, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(whole, staged):
        assert torch.equal(a, b)
    rows = B * H * N
    half = nbytes // 2
    f_dq, f_only = ws_dq.view(torch.float32), ws_only.view(torch.float32)
    # D: two fp32 summation orders of the same d products; each is within
    # d * 2^-24 * sum_k |dO_ik O_ik| of the exact sum (Higham's bound for a
    # recursive sum of products), so they differ by at most twice that.
    x, y = f_dq[:rows].double(), f_only[:rows].double()
    mag = (do.double() * o.double()).abs().sum(dim=-1).reshape(-1)
    ratio = ((x - y).abs() / (2 * d * 2.0 ** -24 * mag + 1e-30)).max().item()
    log(f"    workspace D: dQ pass vs preprocess, max diff / bound = {ratio:.3f}")
    assert ratio <= 1.0
    # L log2(e): the same single fp32 product on both paths.
    off = half // 4
    assert torch.equal(f_dq[off:off + rows], f_only[off:off + rows])
    lse_np = lse.cpu().numpy().reshape(-1).astype(np.float64)
    assert np.allclose(f_only[off:off + rows].cpu().numpy(),
                       lse_np * math.log2(math.e), rtol=1e-6, atol=1e-6)
    got = [t.cpu().numpy().astype(np.float64) for t in pre]
    for b, h in ((0, 0), (B - 1, H - 1)):
        want = oracle.bwd(ref["q"][b, h], ref["k"][b, h], ref["v"][b, h],
                          ref["do"][b, h], 1 / math.sqrt(d), causal, 0)[:3]
        for name, g, r in zip(("dQ", "dK", "dV"), got, want):
            assert_close(g[b, h], r, BF16_MAX, BF16_MEAN, f"{name} head ({b},{h})")

"""Parity of dropout on P (attn_fwd_dropout, attn_bwd_dropout) with the fp64
oracle's dropout routines, through the C ABI.

The keep indicators are integer work and are checked bit-exactly: with Q = 0
every visible key has the same probability, and one-hot values (forward) or
one-hot output gradients (dK/dV pass) turn O or dV into counts of kept
elements, which must equal the counts of the oracle's indicators.  The dQ
pass is checked on structured inputs at a tolerance below the change one
flipped indicator makes.  Random inputs then take the usual bars: O, dQ, dK,
dV max abs <= 2e-2, mean abs <= 2e-3, LSE max abs <= 1e-3.
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


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def keep_of(p):
    return (256 - oracle.dropout_threshold(p)) / 256


def visible(N, causal, window):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = np.ones((N, N), bool)
    if causal:
        vis &= j <= i
    if window:
        vis &= np.abs(i - j) < window
    return vis


def masks(B, H, N, p, seed, offset):
    return np.stack([oracle.dropout_mask(seed, offset, p, bh, N, N) for bh in range(B * H)])


# ------------------------------------------------------------ keep indicators

READBACK = [(2, 3, 1, 128, 128), (1, 2, 2, 64, 64), (2, 2, 1, 300, 64), (1, 4, 2, 333, 128)]


@pytest.mark.parametrize("B,H,Hkv,N,d", READBACK)
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 50)])
@pytest.mark.parametrize("p,seed,offset", [(0.1, 7, 0), (0.5, 2**63 + 12345, 99)])
def test_forward_keep_indicators_are_exact(ea, B, H, Hkv, N, d, causal, window, p, seed,
                                           offset):
    log(f"case: dropout fwd read-back B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} "
        f"window={window} p={p}")
    q = torch.zeros(B, H, N, d, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(B, Hkv, N, d, device="cuda").bfloat16()
    eye = torch.zeros(N, d)
    eye[torch.arange(N), torch.arange(N) % d] = 1.0
    v = eye.expand(B, Hkv, N, d).contiguous().cuda().bfloat16()
    o, lse = ea.attn_fwd_dropout(q, k, v, p, seed, offset, causal=causal, window=window,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    vis = visible(N, causal, window)
    nvis = vis.sum(1).astype(np.float64)
    counts = np.rint(o.cpu().numpy().astype(np.float64) * keep_of(p) * nvis[:, None])
    z = masks(B, H, N, p, seed, offset).reshape(B, H, N, N) * vis
    # count[i, c] = number of kept visible keys j with j % d == c
    want = np.zeros((B, H, N, d))
    for c in range(d):
        want[..., c] = z[..., c::d].sum(-1)
    bad = int((counts != want).sum())
    log(f"    indicator counts differing: {bad} of {want.size}")
    assert bad == 0
    np.testing.assert_allclose(lse.cpu().numpy(), np.broadcast_to(np.log(nvis), lse.shape),
                               atol=1e-5)


@pytest.mark.parametrize("B,H,Hkv,N,d", READBACK)
@pytest.mark.parametrize("p,seed,offset", [(0.1, 3, 5), (0.5, 2**40 + 3, 0)])
def test_dkdv_keep_indicators_are_exact(ea, B, H, Hkv, N, d, p, seed, offset):
    """Q = 0 and dO_i = e_{i mod d}: dV_j[c] = sum over query heads of the group
    and queries i = c (mod d) of Z_ij / keep / N."""
    log(f"case: dropout dkdv read-back B{B} H{H} Hkv{Hkv} N{N} d{d} p={p}")
    q = torch.zeros(B, H, N, d, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(B, Hkv, N, d, device="cuda").bfloat16()
    v = torch.randn(B, Hkv, N, d, device="cuda").bfloat16()
    eye = torch.zeros(N, d)
    eye[torch.arange(N), torch.arange(N) % d] = 1.0
    do = eye.expand(B, H, N, d).contiguous().cuda().bfloat16()
    o, lse = ea.attn_fwd_dropout(q, k, v, p, seed, offset)
    dq, dk, dv = ea.attn_bwd_dropout(q, k, v, o, do, lse, p, seed, offset)
    torch.cuda.synchronize()
    counts = np.rint(dv.cpu().numpy().astype(np.float64) * keep_of(p) * N)
    z = masks(B, H, N, p, seed, offset).reshape(B, Hkv, H // Hkv, N, N).sum(2)
    want = np.zeros((B, Hkv, N, d))  # [.., key j, c]
    for c in range(d):
        want[..., c] = z[..., c::d, :].sum(-2)
    bad = int((counts != want).sum())
    log(f"    indicator counts differing: {bad} of {want.size}")
    assert bad == 0


@pytest.mark.parametrize("B,H,Hkv,N,d", READBACK)
@pytest.mark.parametrize("causal", [False, True])
def test_dq_structured_inputs(ea, B, H, Hkv, N, d, causal):
    """Q = 0, V = 1, dO_i = e_0: dP = 1, P_ij = 1 / n_i over the n_i visible
    keys, so dS_ij = (Z_ij / keep - D_i) / n_i and dQ_i = s sum_j dS_ij K_j.
    One flipped indicator moves component c of dQ_i by s |K_jc| / (keep n_i).
    The bar per element is 2e-4 plus the two roundings the GPU path adds, with
    25 % margin: D_i = O_i[0] is read from the bf16 O (|dD_i| <= 2^-9 |D_i|,
    entering as s |dD_i| |mean of K_jc over the visible keys|), and every dS_ij
    is rounded to bf16 for the matrix core (<= 2^-9 (1 / keep + |D_i|) / n_i
    each, entering as s 2^-9 (1 / keep + |D_i|) mean |K_jc|).  In rows with
    few visible keys (the first rows under the causal mask) a flip moves dQ_i
    by far more than the bar."""
    p, seed, offset = 0.3, 41, 2
    log(f"case: dropout dq structured B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    g = torch.Generator().manual_seed(N + d)
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    k = torch.randn(B, Hkv, N, d, generator=g).bfloat16()
    v = torch.ones(B, Hkv, N, d, dtype=torch.bfloat16)
    do = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    do[..., 0] = 1.0
    dev = [t.cuda() for t in (q, k, v, do)]
    o, lse = ea.attn_fwd_dropout(*dev[:3], p, seed, offset, causal=causal)
    dq, dk, dv = ea.attn_bwd_dropout(*dev[:3], o, dev[3], lse, p, seed, offset,
                                     causal=causal)
    torch.cuda.synchronize()
    ref = [t.double().numpy() for t in (q, k, v, do)]
    s = 1 / math.sqrt(d)
    dq_ref, _, _, D_ref = oracle.bwd_dropout(*ref, s, p, seed, offset, causal=causal)
    vis = visible(N, causal, 0)
    wts = vis / vis.sum(1, keepdims=True)
    krep = np.repeat(ref[1], H // Hkv, axis=1)
    kmean = np.einsum("ij,bhjc->bhic", wts, krep)
    kabs = np.einsum("ij,bhjc->bhic", wts, np.abs(krep))
    aD = np.abs(D_ref)[..., None]
    bar = 2e-4 + 1.25 * s * 2.0 ** -9 * (aD * np.abs(kmean) + (1 / keep_of(p) + aD) * kabs)
    err = np.abs(np64(dq) - dq_ref)
    log(f"    dQ: max_abs={err.max():.3e} max err/bar={(err / bar).max():.3f}")
    assert (err <= bar).all()


# ------------------------------------------------------------ random inputs

CASES = [(2, 4, 4, 333, 128), (1, 4, 2, 257, 64), (2, 3, 3, 100, 64), (1, 4, 1, 65, 128),
         (1, 2, 2, 1000, 128)]
MASKS = [(False, 0), (True, 0), (True, 40), (False, 30)]


@pytest.mark.parametrize("B,H,Hkv,N,d", CASES)
@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("p", [0.1, 0.4])
def test_dropout_forward(ea, B, H, Hkv, N, d, causal, window, p):
    log(f"case: dropout fwd B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} "
        f"window={window} p={p}")
    dev, ref = bf16_case(950 + N, B, H, N, d)
    k, v = dev["k"][:, :Hkv].contiguous(), dev["v"][:, :Hkv].contiguous()
    seed, offset = 1000 + N, 3
    o, lse = ea.attn_fwd_dropout(dev["q"], k, v, p, seed, offset, causal=causal,
                                 window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_dropout(ref["q"], ref["k"][:, :Hkv], ref["v"][:, :Hkv],
                                        1 / math.sqrt(d), p, seed, offset, causal, window)
    assert_close(np64(o), o_ref, BF16_MAX, BF16_MEAN, "O")
    assert_close(np64(lse), lse_ref, LSE_MAX, None, "LSE")


@pytest.mark.parametrize("B,H,Hkv,N,d", CASES)
@pytest.mark.parametrize("causal,window", MASKS[:3])
@pytest.mark.parametrize("p", [0.1, 0.4])
def test_dropout_backward(ea, B, H, Hkv, N, d, causal, window, p):
    log(f"case: dropout bwd B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} "
        f"window={window} p={p}")
    dev, ref = bf16_case(960 + N, B, H, N, d, with_dout=True)
    k, v = dev["k"][:, :Hkv].contiguous(), dev["v"][:, :Hkv].contiguous()
    seed, offset = 77 + N, 11
    o, lse = ea.attn_fwd_dropout(dev["q"], k, v, p, seed, offset, causal=causal,
                                 window=window)
    dq, dk, dv = ea.attn_bwd_dropout(dev["q"], k, v, o, dev["do"], lse, p, seed, offset,
                                     causal=causal, window=window)
    torch.cuda.synchronize()
    want = oracle.bwd_dropout(ref["q"], ref["k"][:, :Hkv], ref["v"][:, :Hkv], ref["do"],
                              1 / math.sqrt(d), p, seed, offset, causal, window)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), want[:3]):
        assert_close(np64(g), r, BF16_MAX, BF16_MEAN, name)


def test_zero_probability_is_the_plain_path(ea):
    dev, _ = bf16_case(990, 2, 4, 300, 128, with_dout=True)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o0, l0 = ea.attn_fwd(q, k, v, causal=True)
    o1, l1 = ea.attn_fwd_dropout(q, k, v, 0.0, 5, causal=True)
    g0 = ea.attn_bwd(q, k, v, o0, do, l0, causal=True)
    g1 = ea.attn_bwd_dropout(q, k, v, o1, do, l1, 0.0, 5, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_dropout_is_deterministic_and_follows_seed_and_offset(ea):
    dev, _ = bf16_case(991, 1, 4, 512, 64, with_dout=True)
    q, k, v = dev["q"], dev["k"], dev["v"]
    a, _ = ea.attn_fwd_dropout(q, k, v, 0.2, 123, 4)
    b, _ = ea.attn_fwd_dropout(q, k, v, 0.2, 123, 4)
    c, _ = ea.attn_fwd_dropout(q, k, v, 0.2, 123, 5)
    e, _ = ea.attn_fwd_dropout(q, k, v, 0.2, 124, 4)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c) and not torch.equal(a, e)


def test_dropout_full_size_sampled(ea):
    """B4 H16 N2048 d128 causal, p = 0.1 (the bf16 training shape): the forward
    of the first and last heads and the backward of the first and last heads,
    against the oracle on those heads with their global head indices."""
    B, H, N, d, p, seed, offset = 4, 16, 2048, 128, 0.1, 2024, 1
    log(f"case: dropout full size B{B} H{H} N{N} d{d} causal p={p}")
    dev, ref = bf16_case(992, B, H, N, d, with_dout=True)
    o, lse = ea.attn_fwd_dropout(dev["q"], dev["k"], dev["v"], p, seed, offset, causal=True)
    dq, dk, dv = ea.attn_bwd_dropout(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, p,
                                     seed, offset, causal=True)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (np64(t) for t in (o, lse, dq, dk, dv))
    s = 1 / math.sqrt(d)
    for b, h in ((0, 0), (B - 1, H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        args = (ref["q"][sl], ref["k"][sl], ref["v"][sl])
        o_r, l_r = oracle.fwd_dropout(*args, s, p, seed, offset, True, bh0=b * H + h)
        assert_close(o[sl], o_r, BF16_MAX, BF16_MEAN, f"O head ({b},{h})")
        assert_close(lse[sl], l_r, LSE_MAX, None, f"LSE head ({b},{h})")
        want = oracle.bwd_dropout(*args, ref["do"][sl], s, p, seed, offset, True,
                                  bh0=b * H + h)
        for name, g, r in zip(("dQ", "dK", "dV"), (dq[sl], dk[sl], dv[sl]), want[:3]):
            assert_close(g, r, BF16_MAX, BF16_MEAN, f"{name} head ({b},{h})")

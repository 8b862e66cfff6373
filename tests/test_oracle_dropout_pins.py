"""Pins for the oracle's dropout: its random numbers and what it does with them.

* the generator: the shared Philox-4xW-R routine against numpy's
  Philox-4x64-10 bit generator (a library implementation of the same
  published generator), its Weyl constants against their closed forms
  (golden ratio, sqrt(3)), and the 4x32 keep bytes against uniformity and
  independence statistics;
* the keep rule: a pure function of (seed, offset, head, query, key), keep
  rate 1 - t/256, t = round(256 p);
* the forward: p = 0 is ordinary attention; Q = 0 with one-hot values reads
  the keep indicators back out of O in closed form; the mean of O over many
  seeds is the undropped O (inverted dropout is unbiased);
* the backward: PyTorch fp64 autograd of softmax(S) * Z / keep @ V with the
  same indicators, fp64 central finite differences of sum(O * dO), and
  D_i = sum_k dO_ik O_ik.

The 32-bit instance itself -- its multipliers, Weyl constants and word
layout -- is pinned word for word against rocRAND's Philox-4x32-10 engine in
test_oracle_philox_rocrand.py; the GPU parity tests then compare the
kernels' keep bytes with the oracle's.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def rnd(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ---------------------------------------------------------------- generator

@pytest.mark.parametrize("case", range(6))
def test_philox4x64_matches_numpy(case):
    g = np.random.Generator(np.random.PCG64(900 + case))
    key = [int(x) for x in g.integers(0, 2**64, size=2, dtype=np.uint64)]
    ctr = [int(x) for x in g.integers(0, 2**64, size=4, dtype=np.uint64)]
    if case == 5:
        ctr[0] = 2**64 - 2  # numpy's increment carries into word 1 on its second block
    # uint64 arrays: numpy would round Python ints above 2**53 through float64.
    bg = np.random.Philox(counter=np.array(ctr, np.uint64), key=np.array(key, np.uint64))
    assert [int(x) for x in bg.state["state"]["counter"]] == ctr
    got = bg.random_raw(8)
    # numpy adds one to the counter (with carry) before each block of four.
    c = ctr[0] + (ctr[1] << 64) + (ctr[2] << 128) + (ctr[3] << 192)
    for blk in range(2):
        cc = (c + 1 + blk) % 2**256
        words = [(cc >> (64 * x)) & (2**64 - 1) for x in range(4)]
        mine = oracle.philox(64, 10, words, key)
        assert [int(x) for x in mine] == [int(x) for x in got[4 * blk:4 * blk + 4]]


def test_philox_weyl_constants_are_their_closed_forms():
    # W0 = frac(golden ratio) and W1 = sqrt(3) - 1, as fixed-point fractions.
    w0_64 = (math.isqrt(5 << 128) - (1 << 64)) // 2
    w1_64 = math.isqrt(3 << 128) - (1 << 64)
    c64 = [int(x) for x in oracle.philox_constants(64)]
    c32 = [int(x) for x in oracle.philox_constants(32)]
    assert c64[2:] == [w0_64, w1_64]
    assert c32[2:] == [w0_64 >> 32, w1_64 >> 32]
    assert all(x < 2**32 for x in c32) and all(x % 2 == 1 for x in c32[:2] + c64[:2])


def test_philox_rounds_mix_every_counter_word():
    # One flipped counter or key bit changes about half of the 128 output bits.
    key = [0x1234, 0x5678]
    base = oracle.philox(32, 10, [1, 2, 3, 4], key)
    flips = []
    for w in range(6):
        for bit in (0, 13, 31):
            c, k = [1, 2, 3, 4], list(key)
            if w < 4:
                c[w] ^= 1 << bit
            else:
                k[w - 4] ^= 1 << bit
            o = oracle.philox(32, 10, c, k)
            flips.append(sum(bin(int(a) ^ int(b)).count("1") for a, b in zip(o, base)))
    assert min(flips) > 40 and max(flips) < 88
    assert abs(np.mean(flips) - 64) < 8


def test_dropout_bytes_are_uniform_and_independent():
    z = np.stack([np.array([[oracle.dropout_byte(77, 3, bh, i, j) for j in range(64)]
                            for i in range(64)]) for bh in range(2)])
    # 8192 bytes: chi-square over 256 bins (255 dof: mean 255, sd 22.6).
    counts = np.bincount(z.ravel(), minlength=256)
    chi2 = ((counts - z.size / 256) ** 2 / (z.size / 256)).sum()
    assert chi2 < 255 + 6 * 22.6
    # Neighbours inside and across 4x4 sub-blocks and across heads agree by chance only.
    for a, b in [(z[:, 1:, :], z[:, :-1, :]), (z[:, :, 1:], z[:, :, :-1]),
                 (z[:, 4:, :], z[:, :-4, :]), (z[:, :, 4:], z[:, :, :-4]), (z[0], z[1])]:
        frac = (a == b).mean()
        assert abs(frac - 1 / 256) < 6 * math.sqrt(a.size / 256) / a.size


def test_dropout_mask_is_a_pure_function_of_its_coordinates():
    full = oracle.dropout_mask(5, 9, 0.3, 7, 40, 50)
    part = oracle.dropout_mask(5, 9, 0.3, 7, 13, 21, i0=17, j0=22)
    np.testing.assert_array_equal(part, full[17:30, 22:43])
    for other in [oracle.dropout_mask(5, 10, 0.3, 7, 40, 50),  # offset
                  oracle.dropout_mask(6, 9, 0.3, 7, 40, 50),   # seed
                  oracle.dropout_mask(5, 9, 0.3, 8, 40, 50)]:  # head
        agree = (other == full).mean()
        assert abs(agree - (0.7 ** 2 + 0.3 ** 2)) < 0.05  # independent draws


@pytest.mark.parametrize("p,t", [(0.0, 0), (0.1, 26), (0.5, 128), (127.5 / 256, 128),
                                 (0.2, 51), (0.99, 253)])
def test_dropout_threshold_rounds_half_up(p, t):
    assert oracle.dropout_threshold(p) == t


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_dropout_keep_rate(p):
    t = oracle.dropout_threshold(p)
    z = oracle.dropout_mask(2024, 0, p, 3, 512, 512)
    q = (256 - t) / 256
    assert abs(z.mean() - q) < 6 * math.sqrt(q * (1 - q) / z.size)


# ---------------------------------------------------------------- forward

MASKS = [(False, 0), (True, 0), (True, 5), (False, 3)]


@pytest.mark.parametrize("causal,window", MASKS)
def test_zero_dropout_is_ordinary_attention(causal, window):
    q, k, v, do = (rnd(40 + x, 1, 2, 37, 8) for x in range(4))
    o, lse = oracle.fwd_dropout(q, k, v, 0.3, 0.0, 11, causal=causal, window=window)
    o0, lse0 = oracle.fwd(q, k, v, 0.3, causal, window)
    np.testing.assert_allclose(o, o0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse0, rtol=0, atol=1e-14)
    g = oracle.bwd_dropout(q, k, v, do, 0.3, 0.0, 11, causal=causal, window=window)
    g0 = oracle.bwd(q, k, v, do, 0.3, causal, window)
    for a, b in zip(g, g0):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,window", MASKS)
def test_uniform_probabilities_read_back_the_keep_indicators(causal, window):
    # Q = 0 makes P uniform over the visible keys; V_j = e_j reads Z_ij / keep
    # / (number visible) into O_i[j].
    B, H, N, d, p = 2, 2, 24, 24, 0.4
    q = np.zeros((B, H, N, d))
    k = rnd(5, B, H, N, d)
    v = np.broadcast_to(np.eye(N, d), (B, H, N, d)).copy()
    o, lse = oracle.fwd_dropout(q, k, v, 0.5, p, 99, 4, causal=causal, window=window)
    keep = (256 - oracle.dropout_threshold(p)) / 256
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = np.ones((N, N), bool)
    if causal:
        vis &= j <= i
    if window:
        vis &= np.abs(i - j) < window
    nvis = vis.sum(1)
    for bh in range(B * H):
        z = oracle.dropout_mask(99, 4, p, bh, N, N) * vis
        np.testing.assert_allclose(o.reshape(B * H, N, d)[bh], z / keep / nvis[:, None],
                                   rtol=1e-14, atol=0)
        np.testing.assert_allclose(lse.reshape(B * H, N)[bh], np.log(nvis), rtol=1e-14)


def test_dropout_is_unbiased_over_seeds():
    q, k, v = (rnd(70 + x, 1, 1, 6, 3) for x in range(3))
    o0, _ = oracle.fwd(q, k, v, 0.7, True, 0)
    S = 3000
    outs = np.stack([oracle.fwd_dropout(q, k, v, 0.7, 0.5, s, causal=True)[0] for s in range(S)])
    mean, sd = outs.mean(0), outs.std(0)
    assert (np.abs(mean - o0) <= 5 * sd / math.sqrt(S) + 1e-12).all()
    # A missing 1/keep factor would give o0 / 2.
    assert np.abs(mean - o0).max() < 0.1 * np.abs(o0).max()


def test_gqa_dropout_equals_repeated_heads():
    q, do = rnd(80, 2, 4, 19, 8), rnd(81, 2, 4, 19, 8)
    k, v = rnd(82, 2, 2, 19, 8), rnd(83, 2, 2, 19, 8)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    o, lse = oracle.fwd_dropout(q, k, v, 0.4, 0.25, 7, 1, causal=True)
    o1, lse1 = oracle.fwd_dropout(q, kr, vr, 0.4, 0.25, 7, 1, causal=True)
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(lse, lse1)
    dq, dk, dv, D = oracle.bwd_dropout(q, k, v, do, 0.4, 0.25, 7, 1, causal=True)
    dq1, dk1, dv1, D1 = oracle.bwd_dropout(q, kr, vr, do, 0.4, 0.25, 7, 1, causal=True)
    np.testing.assert_allclose(dq, dq1, atol=1e-14)
    np.testing.assert_allclose(dk, dk1.reshape(2, 2, 2, 19, 8).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dv1.reshape(2, 2, 2, 19, 8).sum(2), atol=1e-13)


def test_head_offset_numbers_a_slice_like_the_whole():
    q, k, v, do = (rnd(90 + x, 2, 3, 21, 8) for x in range(4))
    o, lse = oracle.fwd_dropout(q, k, v, 0.4, 0.3, 12, 3, causal=True)
    g = oracle.bwd_dropout(q, k, v, do, 0.4, 0.3, 12, 3, causal=True)
    b, h = 1, 2
    sl = (slice(b, b + 1), slice(h, h + 1))
    o1, lse1 = oracle.fwd_dropout(q[sl], k[sl], v[sl], 0.4, 0.3, 12, 3, causal=True,
                                  bh0=b * 3 + h)
    np.testing.assert_array_equal(o1, o[sl])
    np.testing.assert_array_equal(lse1, lse[sl])
    g1 = oracle.bwd_dropout(q[sl], k[sl], v[sl], do[sl], 0.4, 0.3, 12, 3, causal=True,
                            bh0=b * 3 + h)
    for a, r in zip(g1, g):
        np.testing.assert_array_equal(a, r[sl])


# ---------------------------------------------------------------- backward

def torch_dropout_attention(q, k, v, z, keep, scale, causal, window):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).requires_grad_() for x in (q, k, v))
    N = tq.shape[-2]
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    m = torch.ones(N, N, dtype=torch.bool)
    if causal:
        m &= j <= i
    if window > 0:
        m &= (i - j).abs() < window
    s = (tq @ tk.transpose(-1, -2).contiguous()) * scale
    pr = torch.softmax(s.masked_fill(~m, float("-inf")), dim=-1)
    o = (pr * torch.from_numpy(z.astype(np.float64)) / keep) @ tv
    return tq, tk, tv, o


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("p", [0.15, 0.6])
def test_dropout_backward_matches_torch_autograd(causal, window, p):
    B, H, N, d = 1, 3, 29, 8
    q, k, v, do = (rnd(100 + x, B, H, N, d) for x in range(4))
    keep = (256 - oracle.dropout_threshold(p)) / 256
    z = np.stack([oracle.dropout_mask(31, 2, p, bh, N, N) for bh in range(B * H)])
    z = z.reshape(B, H, N, N)
    tq, tk, tv, o = torch_dropout_attention(q, k, v, z, keep, 0.35, causal, window)
    (o * torch.from_numpy(do)).sum().backward()
    mo, _ = oracle.fwd_dropout(q, k, v, 0.35, p, 31, 2, causal=causal, window=window)
    np.testing.assert_allclose(mo, o.detach().numpy(), rtol=0, atol=1e-12)
    dq, dk, dv, D = oracle.bwd_dropout(q, k, v, do, 0.35, p, 31, 2, causal=causal,
                                       window=window)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    # D_i = sum_k dO_ik O_ik with the dropped output.
    np.testing.assert_allclose(D, (do * mo).sum(-1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_backward_finite_differences(causal):
    B, H, Hkv, N, d, p, sc = 1, 2, 1, 7, 3, 0.45, 0.8
    q, do = rnd(120, B, H, N, d), rnd(121, B, H, N, d)
    k, v = rnd(122, B, Hkv, N, d), rnd(123, B, Hkv, N, d)

    def loss(qq, kk, vv):
        return (oracle.fwd_dropout(qq, kk, vv, sc, p, 5, 6, causal=causal)[0] * do).sum()

    grads = oracle.bwd_dropout(q, k, v, do, sc, p, 5, 6, causal=causal)[:3]
    eps = 1e-6
    for x, g in zip((q, k, v), grads):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.abs(num - g).max() <= 1e-7 * max(1.0, np.abs(g).max())

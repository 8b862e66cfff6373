"""Pins for the fp64 oracle: it is checked against things other than itself.

* closed forms that follow from the softmax definition (constant V, identical
  keys, Q = 0, a dominant key, causal edges, window edges);
* invariants (rows of P sum to 1, key shift, permutations, sum_j dK_j = 0,
  D = rowsum(dO * O));
* the pages' decomposition identities (block-wise online softmax, both the
  normalised and the unnormalised accumulator forms, equal the two-pass form);
* an independent library implementation of the same definition: PyTorch's
  CPU scaled_dot_product_attention and its autograd, in float64;
* fp64 central finite differences of sum(O * dO) for the gradients;
* a hand-derived worked example (tests/golden/three_key_worked_example.json);
* the number-format decoders against PyTorch's bf16 / float8_e4m3fn types.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import attn_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def torch_mask(N, causal, window):
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    m = torch.ones(N, N, dtype=torch.bool)
    if causal:
        m &= j <= i
    if window > 0:
        m &= (i - j).abs() < window
    return m


def torch_attention(q, k, v, scale, causal, window):
    """PyTorch fp64 CPU SDPA with an explicit boolean mask; O and LSE."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    N = tq.shape[-2]
    mask = torch_mask(N, causal, window)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, scale=scale)
    s = (tq @ tk.transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


SHAPES = [(1, 1, 4), (2, 17, 8), (1, 33, 16), (3, 64, 4), (1, 70, 32)]
MASKS = [(False, 0), (True, 0), (True, 5), (False, 3), (True, 1), (True, 200)]


# ---------------------------------------------------------------- formats
def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_synth_e4m3_encoder_round_trips_and_rounds_to_nearest_even():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.decode_e4m3(codes)
    assert (attn_synth.e4m3_codes(vals)[vals != 0] == codes[vals != 0]).all()
    # midpoints between neighbours round to the even code
    pos = np.sort(oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2
    enc = oracle.decode_e4m3(attn_synth.e4m3_codes(mids))
    lo_code = attn_synth.e4m3_codes(pos[:-1])
    expect = np.where(lo_code % 2 == 0, pos[:-1], pos[1:])
    assert (enc == expect).all()
    # saturation, and agreement with torch's own conversion inside the range
    assert attn_synth.e4m3_codes(np.array([1e6, -500.0]))[0] == 0x7E
    x = rnd(7, 4096) * 50
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch rounds from fp32; compare only where fp64->fp32 does not move a tie
    ours = attn_synth.e4m3_codes(x.astype(np.float32).astype(np.float64))
    assert (ours == ref).all()


def test_synth_bf16_matches_torch_rounding():
    x = rnd(3, 10000) * 7
    ours = attn_synth.bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert (ours.view(np.int16) == ref).all()


# ---------------------------------------------------------------- forward
@pytest.mark.parametrize("BH,N,d", SHAPES)
@pytest.mark.parametrize("causal,window", MASKS)
def test_forward_matches_torch_sdpa_fp64(BH, N, d, causal, window):
    q, k, v = rnd(1, BH, N, d), rnd(2, BH, N, d), rnd(3, BH, N, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.fwd(q, k, v, scale, causal, window)
    o_ref, lse_ref = torch_attention(q, k, v, scale, causal, window)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_golden_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "three_key_worked_example.json")))
    q, k, v = (np.array(g[n]) for n in ("q", "k", "v"))
    for case in g["cases"]:
        o, lse = oracle.fwd(q, k, v, g["scale"], case["causal"], case["window"])
        np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, case["lse"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("form", [1, 2])
def test_online_block_recurrence_equals_two_pass(causal, window, form):
    N, d = 53, 8
    q, k, v = rnd(11, N, d) * 2, rnd(12, N, d) * 2, rnd(13, N, d)
    o, lse = oracle.fwd(q, k, v, 0.4, causal, window)
    g = np.random.Generator(np.random.PCG64(99))
    for trial in range(6):
        nparts = int(g.integers(1, N + 1))
        cuts = np.sort(g.choice(np.arange(1, N), size=nparts - 1, replace=False))
        bounds = np.concatenate([[0], cuts, [N]])
        o2, lse2 = oracle.online_fwd(q, k, v, bounds, form, 0.4, causal, window)
        assert np.abs(o2 - o).max() <= 1e-12 * max(1.0, np.abs(o).max())
        assert np.abs(lse2 - lse).max() <= 1e-12 * max(1.0, np.abs(lse).max())


@pytest.mark.parametrize("causal,window", MASKS)
def test_probability_rows_sum_to_one_and_respect_mask(causal, window):
    N, d = 41, 8
    q, k, v = rnd(21, N, d), rnd(22, N, d), rnd(23, N, d)
    for i in (0, 1, 20, 40):
        p = oracle.probs_row(q, k, v, i, 0.7, causal, window)
        assert abs(p.sum() - 1.0) <= 1e-14
        vis = np.array([oracle.visible(i, j, causal, window) for j in range(N)])
        assert (p[~vis] == 0).all() and (p[vis] > 0).all()


def n_visible(N, causal, window):
    return np.array([sum(oracle.visible(i, j, causal, window) for j in range(N))
                     for i in range(N)])


@pytest.mark.parametrize("causal,window", MASKS)
def test_constant_values_give_constant_output(causal, window):
    N, d = 37, 16
    q, k = rnd(31, N, d) * 3, rnd(32, N, d) * 3
    c = rnd(33, d)
    v = np.tile(c, (N, 1))
    o, _ = oracle.fwd(q, k, v, 0.5, causal, window)
    np.testing.assert_allclose(o, np.tile(c, (N, 1)), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", MASKS)
def test_identical_keys_give_mean_of_visible_values(causal, window):
    N, d = 29, 8
    q, v = rnd(41, N, d), rnd(43, N, d)
    kv = rnd(42, d)
    k = np.tile(kv, (N, 1))
    s = 0.3
    o, lse = oracle.fwd(q, k, v, s, causal, window)
    cnt = n_visible(N, causal, window)
    for i in range(N):
        vis = [j for j in range(N) if oracle.visible(i, j, causal, window)]
        np.testing.assert_allclose(o[i], v[vis].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[i] - (s * q[i] @ kv + math.log(cnt[i]))) <= 1e-13


@pytest.mark.parametrize("causal,window", MASKS)
def test_zero_queries_give_log_count(causal, window):
    N, d = 31, 4
    q = np.zeros((N, d))
    k, v = rnd(52, N, d), rnd(53, N, d)
    _, lse = oracle.fwd(q, k, v, 1.0, causal, window)
    np.testing.assert_allclose(lse, np.log(n_visible(N, causal, window)), rtol=0, atol=1e-14)


def test_dominant_key_closed_form():
    # S_i = [a, b, b, ..., b] -> P_i0 = e^a / (e^a + (n-1) e^b)
    n, d = 9, 2
    a, b = 2.5, -0.75
    q = np.array([[1.0, 0.0]])
    k = np.zeros((n, d))
    k[0, 0] = a
    k[1:, 0] = b
    v = rnd(61, n, d)
    qq = np.repeat(q, n, axis=0)  # every row has the same scores
    o, lse = oracle.fwd(qq, k, v, 1.0, False, 0)
    p0 = math.exp(a) / (math.exp(a) + (n - 1) * math.exp(b))
    pb = math.exp(b) / (math.exp(a) + (n - 1) * math.exp(b))
    expect = p0 * v[0] + pb * v[1:].sum(axis=0)
    np.testing.assert_allclose(o[0], expect, rtol=0, atol=1e-14)
    assert abs(lse[0] - math.log(math.exp(a) + (n - 1) * math.exp(b))) <= 1e-14
    # a very large gap sends O_i to V_0
    k[0, 0] = 60.0
    o, _ = oracle.fwd(qq, k, v, 1.0, False, 0)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-20 + 1e-12)


def test_causal_and_window_edges():
    N, d = 23, 8
    q, k, v = rnd(71, N, d), rnd(72, N, d), rnd(73, N, d)
    s = 0.35
    o, lse = oracle.fwd(q, k, v, s, True, 0)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert abs(lse[0] - s * q[0] @ k[0]) <= 1e-14
    o1, _ = oracle.fwd(q[:1], k[:1], v[:1], s, False, 0)
    np.testing.assert_allclose(o1, v[:1], rtol=0, atol=1e-15)
    ow, lw = oracle.fwd(q, k, v, s, True, 1)
    np.testing.assert_allclose(ow, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lw, s * np.einsum("nd,nd->n", q, k), rtol=0, atol=1e-14)
    for W in (N, N + 5, 10 * N):
        o2, l2 = oracle.fwd(q, k, v, s, True, W)
        np.testing.assert_array_equal(o2, o)
        np.testing.assert_array_equal(l2, lse)
    # non-causal window >= N is no window at all
    o3, _ = oracle.fwd(q, k, v, s, False, N)
    o4, _ = oracle.fwd(q, k, v, s, False, 0)
    np.testing.assert_array_equal(o3, o4)


def test_key_shift_and_permutation_invariance():
    N, d = 27, 8
    q, k, v = rnd(81, N, d), rnd(82, N, d), rnd(83, N, d)
    s = 0.5
    o, lse = oracle.fwd(q, k, v, s, False, 0)
    u = rnd(84, d)
    o2, lse2 = oracle.fwd(q, k + u, v, s, False, 0)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + s * q @ u, rtol=0, atol=1e-13)
    perm = np.random.Generator(np.random.PCG64(85)).permutation(N)
    o3, lse3 = oracle.fwd(q, k[perm], v[perm], s, False, 0)
    np.testing.assert_allclose(o3, o, rtol=0, atol=1e-13)
    o4, lse4 = oracle.fwd(q[perm], k, v, s, False, 0)
    np.testing.assert_allclose(o4, o[perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse4, lse[perm], rtol=0, atol=1e-13)


def test_fwd_rows_equals_fwd():
    N, d = 45, 16
    q, k, v = rnd(91, N, d), rnd(92, N, d), rnd(93, N, d)
    rows = np.array([0, 3, 44, 17])
    for causal, window in MASKS:
        o, lse = oracle.fwd(q, k, v, 0.25, causal, window)
        o2, lse2 = oracle.fwd_rows(q, k, v, rows, 0.25, causal, window)
        np.testing.assert_array_equal(o2, o[rows])
        np.testing.assert_array_equal(lse2, lse[rows])


# ---------------------------------------------------------------- backward
@pytest.mark.parametrize("BH,N,d", [(1, 5, 3), (2, 19, 8), (1, 40, 16)])
@pytest.mark.parametrize("causal,window", MASKS)
def test_backward_matches_torch_autograd_fp64(BH, N, d, causal, window):
    q, k, v, do = (rnd(100 + t, BH, N, d) for t in range(4))
    s = 1.0 / math.sqrt(d)
    dq, dk, dv, D = oracle.bwd(q, k, v, do, s, causal, window)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch_mask(N, causal, window), scale=s)
    (o * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    # D_i = sum_j P_ij dP_ij equals rowsum(dO * O)
    np.testing.assert_allclose(D, (o.detach().numpy() * do).sum(-1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_backward_finite_differences(causal, window):
    N, d = 7, 3
    q, k, v, do = (rnd(200 + t, N, d) for t in range(4))
    s = 0.8
    dq, dk, dv, _ = oracle.bwd(q, k, v, do, s, causal, window)
    h = 1e-6

    def loss(q_, k_, v_):
        o, _ = oracle.fwd(q_, k_, v_, s, causal, window)
        return float((o * do).sum())

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for i in range(N):
            for c in range(d):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][i, c] += h
                args_m[which][i, c] -= h
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert abs(fd - grad[i, c]) <= 1e-7 * max(1.0, abs(grad[i, c])), (which, i, c)


@pytest.mark.parametrize("causal,window", MASKS)
def test_backward_invariants(causal, window):
    N, d = 33, 8
    q, k, v, do = (rnd(300 + t, N, d) for t in range(4))
    s = 0.6
    dq, dk, dv, D = oracle.bwd(q, k, v, do, s, causal, window)
    # every row of dS sums to zero, so the key gradients sum to zero
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-13)
    # constant V: O does not depend on Q or K
    vc = np.tile(rnd(304, d), (N, 1))
    dq2, dk2, _, _ = oracle.bwd(q, k, vc, do, s, causal, window)
    np.testing.assert_allclose(dq2, 0.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk2, 0.0, rtol=0, atol=1e-13)
    # D identity with the oracle's own O
    o, _ = oracle.fwd(q, k, v, s, causal, window)
    np.testing.assert_allclose(D, (o * do).sum(-1), rtol=0, atol=1e-13)
    # dV columns: sum_j dV_j = sum_i dO_i (each P row sums to 1)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- MQA / GQA
GQA_SHAPES = [(2, 4, 2, 9, 8), (1, 3, 1, 17, 4), (1, 6, 3, 12, 16), (2, 2, 2, 10, 4)]


@pytest.mark.parametrize("B,H,Hkv,N,d", GQA_SHAPES)
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 4), (False, 3)])
def test_gqa_equals_attention_on_repeated_heads(B, H, Hkv, N, d, causal, window):
    """Grouped-query attention is ordinary attention with each key/value head
    repeated for its consecutive query heads (torch fp64 SDPA on the repeated
    tensors), and torch's autograd through the repetition sums the gradients
    of the copies, which is the page's dK, dV accumulation over the group."""
    q, do = rnd(900, B, H, N, d), rnd(901, B, H, N, d)
    k, v = rnd(902, B, Hkv, N, d), rnd(903, B, Hkv, N, d)
    s = 1.0 / math.sqrt(d)
    o, lse = oracle.fwd_gqa(q, k, v, s, causal, window)
    dq, dk, dv, D = oracle.bwd_gqa(q, k, v, do, s, causal, window)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    g = H // Hkv
    kr, vr = tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1)
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, kr, vr, attn_mask=torch_mask(N, causal, window), scale=s)
    (to * torch.from_numpy(do)).sum().backward()
    _, tlse = torch_attention(q, kr.detach().numpy(), vr.detach().numpy(), s, causal,
                              window)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, tlse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(D, (o * do).sum(-1), rtol=0, atol=1e-12)


def test_gqa_with_one_query_head_per_group_is_ordinary_attention():
    B, H, N, d = 2, 3, 11, 8
    q, k, v, do = (rnd(910 + t, B, H, N, d) for t in range(4))
    s = 0.3
    o1, l1 = oracle.fwd_gqa(q, k, v, s, True, 0)
    o2, l2 = oracle.fwd(q, k, v, s, True, 0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    for a, b in zip(oracle.bwd_gqa(q, k, v, do, s, True, 0),
                    oracle.bwd(q, k, v, do, s, True, 0)):
        np.testing.assert_array_equal(a, b)


def test_mqa_shared_head_gradient_is_sum_over_query_heads():
    """With H identical query heads (same q and dO) sharing one key/value
    head, dK and dV are exactly H times those of a single head."""
    N, d, H = 13, 4, 4
    q1, k, v, do1 = (rnd(920 + t, 1, 1, N, d) for t in range(4))
    q, do = np.repeat(q1, H, axis=1), np.repeat(do1, H, axis=1)
    _, dk, dv, _ = oracle.bwd_gqa(q, k, v, do, 0.5, False, 0)
    _, dk1, dv1, _ = oracle.bwd(q1, k, v, do1, 0.5, False, 0)
    np.testing.assert_allclose(dk, H * dk1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dv, H * dv1, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- decode
def torch_mask_rect(Nq, Nk, causal, window):
    """Visibility for queries at positions Nk - Nq .. Nk - 1 against Nk keys."""
    i = torch.arange(Nk - Nq, Nk)[:, None]
    j = torch.arange(Nk)[None, :]
    m = torch.ones(Nq, Nk, dtype=torch.bool)
    if causal:
        m &= j <= i
    if window > 0:
        m &= (i - j).abs() < window
    return m


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d", [(1, 2, 2, 1, 37, 8), (2, 4, 2, 3, 50, 4),
                                             (1, 6, 1, 5, 64, 16), (1, 1, 1, 9, 9, 8)])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 7), (False, 6)])
def test_decode_matches_torch_sdpa(B, H, Hkv, Nq, Nk, d, causal, window):
    """Queries as the last Nq positions of the key sequence: torch fp64 SDPA
    with the rectangular mask, on key/value heads repeated per group."""
    q = rnd(930, B, H, Nq, d)
    k, v = rnd(931, B, Hkv, Nk, d), rnd(932, B, Hkv, Nk, d)
    s = 1.0 / math.sqrt(d)
    o, lse = oracle.fwd_decode(q, k, v, s, causal, window)
    g = H // Hkv
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1)
    mask = torch_mask_rect(Nq, Nk, causal, window)
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                          scale=s)
    ts = (tq @ tk.transpose(-1, -2).contiguous()) * s
    tl = torch.logsumexp(ts.masked_fill(~mask, float("-inf")), dim=-1)
    np.testing.assert_allclose(o, to.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, tl.numpy(), rtol=0, atol=1e-12)


def test_decode_with_full_query_block_is_the_forward():
    B, H, N, d = 1, 2, 23, 8
    q, k, v = (rnd(940 + t, B, H, N, d) for t in range(3))
    for causal, window in ((False, 0), (True, 0), (True, 5)):
        o1, l1 = oracle.fwd_decode(q, k, v, 0.4, causal, window)
        o2, l2 = oracle.fwd(q, k, v, 0.4, causal, window)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_decode_last_rows_of_the_forward():
    """A block of the last Nq queries gives the forward's last Nq rows."""
    B, H, N, d, Nq = 1, 1, 31, 4, 6
    q, k, v = (rnd(950 + t, B, H, N, d) for t in range(3))
    o, lse = oracle.fwd(q, k, v, 0.5, True, 9)
    o2, l2 = oracle.fwd_decode(q[:, :, N - Nq:], k, v, 0.5, True, 9)
    np.testing.assert_array_equal(o2, o[:, :, N - Nq:])
    np.testing.assert_array_equal(l2, lse[:, :, N - Nq:])


# ---------------------------------------------------------------- fp8 blocks
def test_block_decode_matches_per_block_scaling():
    """Block decode = per-tensor decode of each block with its own descale
    (checked against torch's e4m3 conversion)."""
    codes = np.random.Generator(np.random.PCG64(960)).integers(0, 256, (2, 3, 10, 4),
                                                              dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10  # no NaN codes
    ds = np.array([[[0.5, 2.0, 0.25], [1.0, 3.0, 0.125], [4.0, 1.5, 0.75]],
                   [[0.1, 0.2, 0.3], [0.4, 0.5, 0.6], [0.7, 0.8, 0.9]]])
    got = oracle.decode_e4m3_blocks(codes, ds, 4)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(3):
        np.testing.assert_array_equal(got[:, :, 4 * b:4 * b + 4],
                                      t[:, :, 4 * b:4 * b + 4] * ds[:, :, b, None, None])


def test_incoherent_matrix_is_orthogonal_and_keeps_scores():
    for d in (64, 128):
        m = attn_synth.incoherent_matrix(3, d)
        np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-13)
        q, k = rnd(970, 5, d), rnd(971, 7, d)
        np.testing.assert_allclose((q @ m) @ (k @ m).T, q @ k.T, atol=1e-12)
    h = attn_synth.sylvester_hadamard(4)
    np.testing.assert_array_equal(h, [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1],
                                      [1, -1, -1, 1]])

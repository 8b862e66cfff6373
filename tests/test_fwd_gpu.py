"""Parity of the bf16 forward kernel (through the C ABI) against the fp64
oracle, on the same seeded bf16 inputs.

Bars: O max abs <= 2e-2 and mean abs <= 2e-3; LSE max abs <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import (BF16_MAX, BF16_MEAN, LSE_MAX, assert_close, bf16_case, log,
                     to_device_bf16)
import attn_synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import exact_attention_79_amd as ea
    return ea


def run_fwd(ea, dev, causal, window, out_dtype=torch.bfloat16, guard=True):
    """Forward with the outputs carved out of larger buffers whose margins hold
    a sentinel, so any write outside O or LSE is caught."""
    q = dev["q"]
    B, H, N, d = q.shape
    pad = 64
    obuf = torch.full((q.numel() + 2 * pad,), 7.0, device="cuda", dtype=out_dtype)
    lbuf = torch.full((B * H * N + 2 * pad,), 7.0, device="cuda", dtype=torch.float32)
    o = obuf[pad:pad + q.numel()].view(q.shape)
    lse = lbuf[pad:pad + B * H * N].view(B, H, N)
    ea.attn_fwd(q, dev["k"], dev["v"], causal=causal, window=window,
                out_dtype=out_dtype, out=o, lse=lse)
    torch.cuda.synchronize()
    if guard:
        for buf in (obuf, lbuf):
            assert (buf[:pad] == 7.0).all() and (buf[-pad:] == 7.0).all(), \
                "kernel wrote outside its outputs"
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def test_single_head_fp32_output(ea):
    """B=1, H=1, N=256, d=64, non-causal, fp32 O (the smallest workload)."""
    log("case: B1 H1 N256 d64 non-causal fp32")
    dev, ref = bf16_case(1, 1, 1, 256, 64)
    o, lse = run_fwd(ea, dev, False, 0, torch.float32)
    o_ref, lse_ref = oracle.fwd(ref["q"], ref["k"], ref["v"], 1 / 8)
    assert_close(o, o_ref, BF16_MAX, BF16_MEAN, "O")
    assert_close(lse, lse_ref, LSE_MAX, None, "LSE")


SMALL = [(1, 64), (17, 128), (64, 64), (255, 128), (257, 64), (1000, 128), (333, 64)]
MASKS = [(False, 0), (True, 0), (True, 1), (True, 63), (True, 64), (True, 65),
         (False, 65), (True, 10**6)]


@pytest.mark.parametrize("N,d", SMALL)
@pytest.mark.parametrize("causal,window", MASKS)
def test_ragged_shapes_and_masks(ea, N, d, causal, window):
    log(f"case: B2 H3 N{N} d{d} causal={causal} window={window}")
    dev, ref = bf16_case(100 + N, 2, 3, N, d)
    s = 1 / math.sqrt(d)
    o, lse = run_fwd(ea, dev, causal, window)
    o_ref, lse_ref = oracle.fwd(ref["q"], ref["k"], ref["v"], s, causal, window)
    assert_close(o, o_ref, BF16_MAX, BF16_MEAN, "O")
    assert_close(lse, lse_ref, LSE_MAX, None, "LSE")


def sampled_rows(N, rng, extra=8):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, N // 2, N - 129, N - 65, N - 2, N - 1]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(int(x) for x in rng.integers(0, N, extra))
    return np.array(sorted(rows))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sweep_full_size_sampled(ea, d, causal):
    """B=4, H=16, N=2048: two heads compared in full, every head on sampled rows."""
    B, H, N = 4, 16, 2048
    log(f"case: B{B} H{H} N{N} d{d} causal={causal}")
    dev, ref = bf16_case(2, B, H, N, d)
    s = 1 / math.sqrt(d)
    o, lse = run_fwd(ea, dev, causal, 0)
    for b, h in ((0, 0), (B - 1, H - 1)):
        o_ref, lse_ref = oracle.fwd(ref["q"][b, h], ref["k"][b, h], ref["v"][b, h], s, causal)
        assert_close(o[b, h], o_ref, BF16_MAX, BF16_MEAN, f"O head ({b},{h})")
        assert_close(lse[b, h], lse_ref, LSE_MAX, None, f"LSE head ({b},{h})")
    rng = np.random.default_rng(5)
    got, want, gl, wl = [], [], [], []
    for b in range(B):
        for h in range(H):
            rows = sampled_rows(N, rng, 4)
            o_ref, lse_ref = oracle.fwd_rows(ref["q"][b, h], ref["k"][b, h],
                                             ref["v"][b, h], rows, s, causal)
            got.append(o[b, h][rows]); want.append(o_ref)
            gl.append(lse[b, h][rows]); wl.append(lse_ref)
    assert_close(np.concatenate(got), np.concatenate(want), BF16_MAX, BF16_MEAN,
                 "O sampled rows, all heads")
    assert_close(np.concatenate(gl), np.concatenate(wl), LSE_MAX, None, "LSE sampled")


@pytest.mark.parametrize("N,d", [(600, 128), (700, 64)])
@pytest.mark.parametrize("causal,window", MASKS)
def test_small_grid_single_head(ea, N, d, causal, window):
    """One head short enough for fewer than four 256-query workgroups: the
    forward then runs 128-query workgroups (ragged tail), under every mask."""
    log(f"case: B1 H1 N{N} d{d} causal={causal} window={window} (small grid)")
    dev, ref = bf16_case(520 + N, 1, 1, N, d)
    o, lse = run_fwd(ea, dev, causal, window)
    o_ref, lse_ref = oracle.fwd(ref["q"], ref["k"], ref["v"], 1 / math.sqrt(d), causal, window)
    assert_close(o, o_ref, BF16_MAX, BF16_MEAN, "O")
    assert_close(lse, lse_ref, LSE_MAX, None, "LSE")


@pytest.mark.parametrize("d", [64, 128])
def test_closed_form_invariants(ea, d):
    """Constant V -> O = V; window 1 -> O = V; identical keys -> running mean of
    V and LSE = s q.k + ln(#visible); Q = 0 -> LSE = ln(#visible)."""
    N = 300
    log(f"case: invariants N{N} d{d}")
    bits = attn_synth.bf16_attention_inputs(200 + d, 1, 2, N, d)
    q, k, v = (to_device_bf16(bits[n]) for n in ("q", "k", "v"))
    vals = oracle.decode_bf16(bits["v"])
    s = 1 / math.sqrt(d)
    vc = v[:, :, :1, :].expand(-1, -1, N, -1).contiguous()
    o, _ = ea.attn_fwd(q, k, vc, causal=True, out_dtype=torch.float32)
    # P is rounded to bf16 for the P V product while l sums the fp32 values,
    # so O = V up to one bf16 rounding of the weights (relative 2^-8).
    rel = ((o - vc.float()).abs() / vc.float().abs().clamp_min(1e-3)).max().item()
    log(f"    constant V: max relative deviation {rel:.2e}")
    assert rel <= 2.0 ** -8
    o, lse = ea.attn_fwd(q, k, v, causal=True, window=1)
    assert torch.equal(o, v), "window 1 must give O = V exactly"
    kc = k[:, :, :1, :].expand(-1, -1, N, -1).contiguous()
    o, lse = ea.attn_fwd(q, kc, v, causal=True, out_dtype=torch.float32)
    run_mean = np.cumsum(vals, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert_close(o.cpu().numpy(), run_mean, BF16_MAX, BF16_MEAN, "identical keys O")
    qd, kd = oracle.decode_bf16(bits["q"]), oracle.decode_bf16(bits["k"])
    expect = s * np.einsum("bhnd,bhd->bhn", qd, kd[:, :, 0, :]) + np.log(np.arange(1, N + 1))
    assert_close(lse.cpu().numpy(), expect, LSE_MAX, None, "identical keys LSE")
    qz = torch.zeros_like(q)
    _, lse = ea.attn_fwd(qz, k, v, causal=False)
    assert_close(lse.cpu().numpy(), np.full((1, 2, N), math.log(N)), 1e-5, None, "Q=0 LSE")


def test_deterministic_and_stream_respecting(ea):
    log("case: determinism + side stream, B2 H4 N1111 d128 causal")
    dev, _ = bf16_case(300, 2, 4, 1111, 128)
    o1, l1 = ea.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2, l2 = ea.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("N,d", [(512, 128), (700, 128), (512, 64), (700, 64)])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (False, 100)])
def test_two_pipelines_agree_bitwise(ea, N, d, causal, window):
    """The same head through both forward pipelines: alone (fewer than four
    256-query workgroups: free-running waves, one barrier per tile) and as one
    head of a larger launch (the ping-pong kernel: lockstep half-steps).  They
    do the same arithmetic in the same order on differently scheduled LDS
    rings, so any race in either ring shows up as a bit difference."""
    log(f"case: two pipelines, N{N} d{d} causal={causal} window={window}")
    dev, _ = bf16_case(700 + N + d, 2, 4, N, d)
    q, k, v = dev["q"], dev["k"], dev["v"]
    names = (ea.kernel_name(ea.STAGE_FWD, 1, 1, N, d, causal, window),
             ea.kernel_name(ea.STAGE_FWD, 2, 4, N, d, causal, window))
    assert "fwd_bf16_kernel" in names[0] and "fwd_pp_kernel" in names[1], names
    o_all, l_all = ea.attn_fwd(q, k, v, causal=causal, window=window)
    b, h = 1, 2
    o_one, l_one = ea.attn_fwd(q[b:b + 1, h:h + 1].contiguous(), k[b:b + 1, h:h + 1].contiguous(),
                               v[b:b + 1, h:h + 1].contiguous(), causal=causal, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o_one[0, 0], o_all[b, h]) and torch.equal(l_one[0, 0], l_all[b, h])

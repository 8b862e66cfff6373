"""fp8 forward with block quantisation and incoherent processing (FLASH-ATTN
page, FlashAttention-3 summary, the two techniques for FP8 accuracy).

Parity: attn_fwd_fp8_blocks against the fp64 oracle on the block-dequantised
(and, with incoherent processing, transformed) inputs exactly as the kernel
receives them; bars as for the fp8 forward (O max abs <= 1e-1; LSE within
the bound derived from the precision of the scores).

Accuracy: against exact attention of the original, unquantised fp64 inputs
(Q, K, V ~ N(0,1) with one x10 outlier channel), the two techniques must
reduce the RMS error of O and of the LSE (the page reports a 2.6x lower
quantisation error).
"""
import math

import numpy as np
import pytest
import torch

import attn_synth
import oracle
from helpers import FP8_MAX, assert_close, log, to_device_u8
from test_fp8_gpu import assert_lse, fp8_lse_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import exact_attention_79_amd as ea
    return ea


def dequantised(f8, blocks):
    if blocks:
        return {n: oracle.decode_e4m3_blocks(f8[n], f8[n + "_descale"], r)
                for n, r in (("q", 128), ("k", 64), ("v", 64))}
    return {n: oracle.decode_e4m3(f8[n], f8[n + "_descale"]) for n in ("q", "k", "v")}


def run_gpu(ea, f8, blocks, causal, window=0, Hkv=None):
    dev = {n: to_device_u8(f8[n]) for n in ("q", "k", "v")}
    if blocks:
        ds = {n: torch.from_numpy(np.ascontiguousarray(f8[n + "_descale"], np.float32)).cuda()
              for n in ("q", "k", "v")}
        o, lse = ea.attn_fwd_fp8_blocks(dev["q"], dev["k"], dev["v"], ds["q"], ds["k"],
                                        ds["v"], causal=causal, window=window)
    else:
        o, lse = ea.attn_fwd_fp8(dev["q"], dev["k"], dev["v"], f8["q_descale"],
                                 f8["k_descale"], f8["v_descale"], causal=causal,
                                 window=window)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("N,causal,window", [(1000, False, 0), (777, True, 0),
                                             (300, True, 100), (64, False, 0)])
@pytest.mark.parametrize("incoherent", [False, True])
def test_block_parity(ea, N, causal, window, incoherent):
    B, H, d = 1, 3, 128
    log(f"case: fp8 blocks B{B} H{H} N{N} d{d} causal={causal} window={window} "
        f"incoherent={incoherent}")
    f8 = attn_synth.fp8_attention_inputs_v2(980, B, H, N, d, blocks=True,
                                            incoherent=incoherent)
    ref = dequantised(f8, True)
    s = 1 / math.sqrt(d)
    o, lse = run_gpu(ea, f8, True, causal, window)
    o_ref, l_ref = oracle.fwd(ref["q"], ref["k"], ref["v"], s, causal, window)
    assert_close(o, o_ref, FP8_MAX, None, "O")
    for h in range(H):
        assert_lse(lse[0, h], l_ref[0, h],
                   fp8_lse_bound(ref["q"][0, h], ref["k"][0, h], s, causal, window),
                   f"LSE head {h}")


def test_block_entry_with_uniform_descales_equals_per_tensor(ea):
    """Every block carrying the tensor's descale gives attn_fwd_fp8's result up
    to the rounding of the weights' exponent argument (the block path folds
    the value descale into it; the per-tensor path applies it at the end)."""
    B, H, N, d = 1, 2, 500, 128
    f8 = attn_synth.fp8_attention_inputs_v2(981, B, H, N, d)
    f8["v_descale"] = 2.0 ** round(math.log2(f8["v_descale"]))
    o1, l1 = run_gpu(ea, f8, False, True)
    fb = dict(f8)
    for n, r in (("q", 128), ("k", 64), ("v", 64)):
        fb[n + "_descale"] = np.full((B, H, (N + r - 1) // r), f8[n + "_descale"])
    o2, l2 = run_gpu(ea, fb, True, True)
    do, dl = np.abs(o1 - o2), np.abs(l1 - l2)
    log(f"    per-tensor vs uniform blocks: O max {do.max():.3e} mean {do.mean():.3e}, "
        f"LSE max {dl.max():.3e}")
    assert do.max() <= 2e-2 and do.mean() <= 1e-4 and dl.max() <= 1e-5


def test_techniques_reduce_error_against_unquantised_attention(ea):
    B, H, N, d = 1, 4, 2048, 128
    s = 1 / math.sqrt(d)
    errs = {}
    for blocks, inc in ((False, False), (True, False), (False, True), (True, True)):
        f8 = attn_synth.fp8_attention_inputs_v2(982, B, H, N, d, blocks=blocks,
                                                incoherent=inc)
        if blocks:
            o, lse = run_gpu(ea, f8, True, False)
        else:
            o, lse = run_gpu(ea, f8, False, False)
        o_ex, l_ex = oracle.fwd(f8["q_in"], f8["k_in"], f8["v_in"], s, False, 0)
        errs[(blocks, inc)] = (float(np.sqrt(((o - o_ex) ** 2).mean())),
                               float(np.sqrt(((lse - l_ex) ** 2).mean())))
        log(f"    blocks={blocks} incoherent={inc}: O rms err {errs[(blocks, inc)][0]:.3e} "
            f"LSE rms err {errs[(blocks, inc)][1]:.3e}")
    base, both = errs[(False, False)], errs[(True, True)]
    log(f"    reduction with both techniques: O {base[0] / both[0]:.2f}x, "
        f"LSE {base[1] / both[1]:.2f}x")
    assert base[0] / both[0] >= 2.0 and base[1] / both[1] >= 2.0


@pytest.mark.parametrize("d,causal,window", [(128, False, 0), (128, True, 0), (128, True, 100),
                                             (64, False, 0), (64, True, 0)])
def test_block_parity_grouped_query(ea, d, causal, window):
    """Block descales with grouped-query K/V (8 query heads on 2 key/value
    heads): each query head reads the K/V blocks and the block descales of
    its own key/value head."""
    B, H, Hkv, N = 1, 8, 2, 700
    log(f"case: fp8 blocks gqa B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} window={window}")
    f8 = attn_synth.fp8_attention_inputs_v2(983, B, H, N, d, blocks=True)
    for n in ("k", "v"):
        f8[n] = np.ascontiguousarray(f8[n][:, :Hkv])
        f8[n + "_descale"] = np.ascontiguousarray(f8[n + "_descale"][:, :Hkv])
    ref = dequantised(f8, True)
    s = 1 / math.sqrt(d)
    o, lse = run_gpu(ea, f8, True, causal, window)
    o_ref, l_ref = oracle.fwd_gqa(ref["q"], ref["k"], ref["v"], s, causal, window)
    assert_close(o, o_ref, FP8_MAX, None, "O")
    G = H // Hkv
    for h in range(H):
        assert_lse(lse[0, h], l_ref[0, h],
                   fp8_lse_bound(ref["q"][0, h], ref["k"][0, h // G], s, causal, window),
                   f"LSE head {h}")

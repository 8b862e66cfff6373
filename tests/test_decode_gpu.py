"""Parity of the decode path (attn_fwd_decode: a block of N_q queries that are
the last N_q positions of N_k keys, split over the keys and merged) against
the fp64 oracle's oracle_fwd_decode, through the C ABI.

Inputs: seeded bf16 N(0,1) tensors (queries and keys from different seeds).
Bars as for the forward: O max abs <= 2e-2, mean abs <= 2e-3; LSE <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import attn_synth
import oracle
from helpers import BF16_MAX, BF16_MEAN, LSE_MAX, assert_close, log, to_device_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import exact_attention_79_amd as ea
    return ea


def decode_case(seed, B, H, Hkv, Nq, Nk, d):
    qb = attn_synth.bf16_attention_inputs(seed, B, H, Nq, d)["q"]
    kv = attn_synth.bf16_attention_inputs(seed + 1, B, Hkv, Nk, d)
    dev = {"q": to_device_bf16(qb), "k": to_device_bf16(kv["k"]),
           "v": to_device_bf16(kv["v"])}
    ref = {"q": oracle.decode_bf16(qb), "k": oracle.decode_bf16(kv["k"]),
           "v": oracle.decode_bf16(kv["v"])}
    return dev, ref


CASES = [
    # B, H, Hkv, Nq, Nk, d, causal, window
    (2, 8, 2, 1, 4099, 128, False, 0),
    (2, 8, 2, 1, 4099, 128, True, 0),
    (1, 4, 1, 4, 1000, 64, True, 0),
    (1, 8, 8, 16, 777, 128, True, 300),
    (1, 16, 2, 5, 333, 64, False, 50),
    (1, 2, 2, 33, 64, 128, True, 0),
    (1, 2, 1, 100, 100, 64, True, 0),
    (3, 4, 4, 2, 31, 128, False, 0),
    (1, 1, 1, 1, 1, 64, True, 0),
    (1, 32, 8, 1, 16384, 128, False, 0),
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,window", CASES)
def test_decode_matches_oracle(ea, B, H, Hkv, Nq, Nk, d, causal, window):
    log(f"case: decode B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal} "
        f"window={window}")
    dev, ref = decode_case(1000 + Nk, B, H, Hkv, Nq, Nk, d)
    o, lse = ea.attn_fwd_decode(dev["q"], dev["k"], dev["v"], causal=causal, window=window)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd_decode(ref["q"], ref["k"], ref["v"], 1 / math.sqrt(d),
                                     causal, window)
    assert_close(o.float().cpu().numpy(), o_ref, BF16_MAX, BF16_MEAN, "O")
    assert_close(lse.cpu().numpy(), l_ref, LSE_MAX, None, "LSE")


def test_decode_fp32_output_and_determinism(ea):
    B, H, Hkv, Nq, Nk, d = 2, 8, 4, 3, 5000, 128
    log(f"case: decode fp32 out B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d}")
    dev, ref = decode_case(1100, B, H, Hkv, Nq, Nk, d)
    a = ea.attn_fwd_decode(dev["q"], dev["k"], dev["v"], causal=True,
                           out_dtype=torch.float32)
    b = ea.attn_fwd_decode(dev["q"], dev["k"], dev["v"], causal=True,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    o_ref, _ = oracle.fwd_decode(ref["q"], ref["k"], ref["v"], 1 / math.sqrt(d), True, 0)
    # fp32 output: only the bf16 rounding of P is left (no output rounding)
    assert_close(a[0].cpu().numpy(), o_ref, 5e-3, 5e-4, "O fp32")


def test_decode_workspace_contents_do_not_matter(ea):
    B, H, Hkv, Nq, Nk, d = 1, 4, 2, 2, 3000, 64
    dev, _ = decode_case(1200, B, H, Hkv, Nq, Nk, d)
    n = ea.attn_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d)
    ws1 = torch.zeros(n, device="cuda", dtype=torch.uint8)
    ws2 = torch.full((n,), 0x7F, device="cuda", dtype=torch.uint8)
    a = ea.attn_fwd_decode(dev["q"], dev["k"], dev["v"], workspace=ws1)
    b = ea.attn_fwd_decode(dev["q"], dev["k"], dev["v"], workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])

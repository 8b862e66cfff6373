"""Shared test helpers: device tensors from the seeded generator, oracle inputs
decoded from the same bits, and the error statistics used by the bars."""
from __future__ import annotations

import sys

import numpy as np

import attn_synth
import oracle

# Bars (max abs, mean abs) against the fp64 oracle.
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
LSE_MAX = 1e-3
FP8_MAX = 1e-1


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()


def to_device_u8(codes: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


def bf16_case(workload: int, B: int, H: int, N: int, d: int, with_dout=False):
    """Bits, device tensors and fp64 oracle inputs for one bf16 case."""
    bits = attn_synth.bf16_attention_inputs(workload, B, H, N, d, with_dout)
    dev = {k: to_device_bf16(v) for k, v in bits.items()}
    ref = {k: oracle.decode_bf16(v) for k, v in bits.items()}
    return dev, ref


def err_stats(got: np.ndarray, ref: np.ndarray):
    e = np.abs(np.asarray(got, np.float64) - ref)
    return float(e.max()) if e.size else 0.0, float(e.mean()) if e.size else 0.0


def assert_close(got, ref, max_abs, mean_abs=None, what=""):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    mx, mn = err_stats(got, ref)
    log(f"    {what}: max_abs={mx:.3e} mean_abs={mn:.3e}")
    assert mx <= max_abs, f"{what}: max abs error {mx:.3e} > {max_abs:.1e}"
    if mean_abs is not None:
        assert mn <= mean_abs, f"{what}: mean abs error {mn:.3e} > {mean_abs:.1e}"

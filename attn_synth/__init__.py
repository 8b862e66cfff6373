"""Seeded synthetic inputs for exact attention.

This module is shared by the tests, the benchmark and the oracle's callers.  It
holds none of the attention arithmetic: it draws N(0,1) samples, rounds them to
the storage formats the library consumes (bf16, OCP e4m3 with a per-tensor
descale) and returns the raw bit patterns.  Every consumer receives the same
bits; the oracle decodes them with its own decoder.

Seeds: tensor t of workload c uses seed ``1000 * c + t`` with t = 0 (Q), 1 (K),
2 (V), 3 (dO), 4 (choice of outlier channels).  Workloads that differ only in
head dim, causal flag or window share seeds.  Samples are drawn in fp64 by
numpy's PCG64 generator, in [B, H, N, d] row-major order.
"""
from __future__ import annotations

import numpy as np

T_Q, T_K, T_V, T_DO, T_OUTLIER, T_SIGNS = 0, 1, 2, 3, 4, 5
E4M3_MAX = 448.0


def seed_of(workload: int, tensor: int) -> int:
    return 1000 * int(workload) + int(tensor)


def normal(seed: int, shape) -> np.ndarray:
    """fp64 N(0,1) samples from PCG64(seed)."""
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def bf16_bits(x) -> np.ndarray:
    """Round to bf16 (nearest, ties to even) and return uint16 bit patterns.

    The value is first rounded to binary32 (numpy's cast, nearest-even), then
    the low 16 bits of the binary32 pattern are rounded away, ties to even.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def e4m3_codes(x) -> np.ndarray:
    """Encode fp64 values as OCP e4m3 ("fn") codes: nearest, ties to even,
    magnitudes at or above 448 saturate to 448 (code 0x7E / 0xFE)."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    out = np.zeros(x.shape, np.uint8)
    sat = a >= E4M3_MAX
    # Subnormal range (below 2^-6): grid step 2^-9, code = multiple of the step.
    sub = (a < 2.0 ** -6) & ~sat
    m_sub = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)  # 0..8; 8 == code 0x08 = 2^-6
    out[sub] = m_sub.astype(np.uint8)
    nrm = ~sub & ~sat
    an = a[nrm]
    _, ex = np.frexp(an)          # an = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1   # an in [2^e, 2^(e+1))
    step = np.ldexp(1.0, e - 3)
    qm = np.rint(an / step).astype(np.int64)  # 8..16
    carry = qm == 16
    e = np.where(carry, e + 1, e)
    qm = np.where(carry, 8, qm)
    code = ((e + 7) << 3) | (qm - 8)
    code = np.minimum(code, 0x7E)
    out[nrm] = code.astype(np.uint8)
    out[sat] = 0x7E
    return out | sign


def bf16_attention_inputs(workload: int, B: int, H: int, N: int, d: int,
                          with_dout: bool = False) -> dict:
    """Q, K, V (and dO) as bf16 bit patterns, shape [B, H, N, d], dtype uint16."""
    shape = (B, H, N, d)
    out = {"q": bf16_bits(normal(seed_of(workload, T_Q), shape)),
           "k": bf16_bits(normal(seed_of(workload, T_K), shape)),
           "v": bf16_bits(normal(seed_of(workload, T_V), shape))}
    if with_dout:
        out["do"] = bf16_bits(normal(seed_of(workload, T_DO), shape))
    return out


def outlier_channels(workload: int, d: int, fraction: float = 0.01) -> np.ndarray:
    """max(1, round(fraction * d)) distinct channel indices chosen by seed."""
    n = max(1, int(round(fraction * d)))
    rng = np.random.Generator(np.random.PCG64(seed_of(workload, T_OUTLIER)))
    return np.sort(rng.choice(d, size=n, replace=False))


def fp8_attention_inputs(workload: int, B: int, H: int, N: int, d: int,
                         outlier_scale: float = 10.0,
                         outlier_fraction: float = 0.01) -> dict:
    """Q, K, V drawn N(0,1) in fp64, the same outlier channels of all three
    multiplied by ``outlier_scale``, then quantised per tensor:
    descale = amax / 448, code = e4m3(x / descale).  Returns codes (uint8,
    [B, H, N, d]) and the three descales (python floats)."""
    shape = (B, H, N, d)
    ch = outlier_channels(workload, d, outlier_fraction)
    out = {"channels": ch}
    for name, t in (("q", T_Q), ("k", T_K), ("v", T_V)):
        x = normal(seed_of(workload, t), shape)
        if outlier_scale != 1.0:
            x[..., ch] *= outlier_scale
        amax = float(np.abs(x).max())
        descale = amax / E4M3_MAX if amax > 0 else 1.0
        out[name] = e4m3_codes(x / descale)
        out[name + "_descale"] = descale
    return out


def sylvester_hadamard(d: int) -> np.ndarray:
    """The d x d Hadamard matrix of Sylvester's construction (d a power of 2):
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    assert d >= 1 and d & (d - 1) == 0
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def incoherent_matrix(workload: int, d: int) -> np.ndarray:
    """A random orthogonal d x d matrix M = diag(s) H_d / sqrt(d) with seeded
    random signs s (the randomness of incoherent processing, drawn here and
    handed to both sides as part of the inputs)."""
    rng = np.random.Generator(np.random.PCG64(seed_of(workload, T_SIGNS)))
    signs = rng.choice(np.array([-1.0, 1.0]), size=d)
    return signs[:, None] * sylvester_hadamard(d) / np.sqrt(d)


def _quantise_rows(x: np.ndarray, block_rows):
    """e4m3 codes of x [..., R, d]: one descale per tensor (block_rows None)
    or per block of block_rows rows of each head, descale = amax / 448."""
    if block_rows is None:
        amax = float(np.abs(x).max())
        descale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
        return e4m3_codes(x / descale), descale
    R = x.shape[-2]
    nblk = (R + block_rows - 1) // block_rows
    descales = np.empty(x.shape[:-2] + (nblk,), np.float64)
    codes = np.empty(x.shape, np.uint8)
    for b in range(nblk):
        blk = x[..., b * block_rows:(b + 1) * block_rows, :]
        amax = np.abs(blk).max(axis=(-2, -1))
        # fp32-representable, as the kernel receives them
        ds = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32).astype(np.float64)
        descales[..., b] = ds
        codes[..., b * block_rows:(b + 1) * block_rows, :] = e4m3_codes(blk / ds[..., None, None])
    return codes, descales


def fp8_attention_inputs_v2(workload: int, B: int, H: int, N: int, d: int,
                            blocks: bool = False, incoherent: bool = False,
                            outlier_scale: float = 10.0,
                            outlier_fraction: float = 0.01) -> dict:
    """The fp64 Q, K, V of fp8_attention_inputs (same seeds and outlier
    channels), optionally with incoherent processing (Q and K multiplied by
    incoherent_matrix before quantising), quantised per tensor or per block
    (128 query rows, 64 key/value rows of each head; descales fp64 arrays).
    Returns the codes, the descales and the original fp64 tensors ("q_in",
    "k_in", "v_in") for measuring the error against unquantised attention."""
    shape = (B, H, N, d)
    ch = outlier_channels(workload, d, outlier_fraction)
    out = {"channels": ch}
    m = incoherent_matrix(workload, d) if incoherent else None
    for name, t, rows in (("q", T_Q, 128), ("k", T_K, 64), ("v", T_V, 64)):
        x = normal(seed_of(workload, t), shape)
        if outlier_scale != 1.0:
            x[..., ch] *= outlier_scale
        out[name + "_in"] = x
        if m is not None and name in ("q", "k"):
            x = x @ m
        out[name], out[name + "_descale"] = _quantise_rows(x, rows if blocks else None)
    return out

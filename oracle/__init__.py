"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``exact_attention_79_amd``) never imports it and the two share no code.

The arithmetic lives in ``attn_oracle.c`` (plain fp64 loops, OpenMP over
rows); this module only marshals numpy arrays through ctypes.  What each
routine computes, and which passage of the pages it follows, is written in
the C file's comments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off keeps every fp64 multiply and add separately rounded, so
# the oracle gives the same bits on any x86-64 host it is run on.
CFLAGS = ["-O3", "-march=x86-64-v2", "-ffp-contract=off", "-fopenmp",
          "-shared", "-fPIC", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile attn_oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i, lg, d = ctypes.c_int, ctypes.c_long, ctypes.c_double
        L.oracle_bf16_decode.argtypes = [ctypes.c_void_p, dp, lg]
        L.oracle_e4m3_decode.argtypes = [ctypes.c_void_p, d, dp, lg]
        L.oracle_e4m3_decode_blocks.argtypes = [ctypes.c_void_p, lg, lg, i, i, dp, dp]
        L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f64.restype = d
        L.oracle_visible.argtypes = [lg, lg, i, lg]
        L.oracle_visible.restype = i
        L.oracle_fwd.argtypes = [i, i, i, d, i, lg, dp, dp, dp, dp, dp, i]
        L.oracle_fwd_rows.argtypes = [i, i, d, i, lg, dp, dp, dp,
                                      ctypes.POINTER(lg), i, dp, dp, i]
        L.oracle_probs_row.argtypes = [i, i, d, i, lg, dp, dp, dp, lg, dp]
        L.oracle_bwd.argtypes = [i, i, i, d, i, lg, dp, dp, dp, dp, dp, dp, dp, dp, i]
        L.oracle_online_fwd.argtypes = [i, i, d, i, lg, dp, dp, dp,
                                        ctypes.POINTER(lg), i, i, dp, dp]
        L.oracle_fwd_gqa.argtypes = [i, i, i, i, i, d, i, lg, dp, dp, dp, dp, dp, i]
        L.oracle_fwd_decode.argtypes = [i, i, i, i, i, i, d, i, lg, dp, dp, dp, dp, dp, i]
        L.oracle_bwd_gqa.argtypes = [i, i, i, i, i, d, i, lg, dp, dp, dp, dp, dp, dp,
                                     dp, dp, i]
        u64, u32 = ctypes.c_uint64, ctypes.c_uint32
        pu64 = ctypes.POINTER(ctypes.c_uint64)
        L.oracle_philox.argtypes = [i, i, pu64, pu64, pu64]
        L.oracle_philox_constants.argtypes = [i, pu64]
        L.oracle_dropout_threshold.argtypes = [d]
        L.oracle_dropout_threshold.restype = i
        L.oracle_dropout_byte.argtypes = [u64, u32, lg, lg, lg]
        L.oracle_dropout_byte.restype = i
        L.oracle_dropout_mask.argtypes = [u64, u32, i, lg, lg, lg, lg, lg, ctypes.c_void_p]
        L.oracle_fwd_dropout.argtypes = [i, i, i, i, i, d, i, lg, d, u64, u32, lg,
                                         dp, dp, dp, dp, dp, i]
        L.oracle_bwd_dropout.argtypes = [i, i, i, i, i, d, i, lg, d, u64, u32, lg,
                                         dp, dp, dp, dp, dp, dp, dp, dp, i]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().oracle_bf16_decode(bits.ctypes.data, _p(out), bits.size)
    return out


def decode_e4m3(codes: np.ndarray, descale: float = 1.0) -> np.ndarray:
    """OCP e4m3 codes (uint8) -> code value * descale, in fp64."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float64)
    lib().oracle_e4m3_decode(codes.ctypes.data, float(descale), _p(out), codes.size)
    return out


def decode_e4m3_blocks(codes: np.ndarray, descales: np.ndarray, block_rows: int) -> np.ndarray:
    """e4m3 codes [..., R, d] with one descale per block of block_rows rows of
    each head (descales [..., ceil(R / block_rows)]) -> exact fp64 values."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    R, d = codes.shape[-2:]
    heads = int(np.prod(codes.shape[:-2])) if codes.ndim > 2 else 1
    ds = _f64(descales)
    assert ds.shape == codes.shape[:-2] + ((R + block_rows - 1) // block_rows,)
    out = np.empty(codes.shape, np.float64)
    lib().oracle_e4m3_decode_blocks(codes.ctypes.data, heads, R, d, block_rows, _p(ds),
                                    _p(out))
    return out


def visible(i: int, j: int, causal: bool, window: int) -> bool:
    return bool(lib().oracle_visible(i, j, int(causal), int(window)))


def fwd(q, k, v, scale: float, causal: bool = False, window: int = 0,
        nthreads: int = 0):
    """O and L (natural-log LSE of the scaled scores) for tensors [..., N, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    assert q.shape == k.shape == v.shape and q.ndim >= 2
    N, d = q.shape[-2:]
    BH = int(np.prod(q.shape[:-2])) if q.ndim > 2 else 1
    o = np.empty_like(q)
    lse = np.empty(q.shape[:-1], np.float64)
    lib().oracle_fwd(BH, N, d, float(scale), int(causal), int(window),
                     _p(q), _p(k), _p(v), _p(o), _p(lse), int(nthreads))
    return o, lse


def fwd_rows(q, k, v, rows, scale: float, causal: bool = False, window: int = 0,
             nthreads: int = 0):
    """O and L for the listed query rows of ONE head (q, k, v: [N, d])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.ndim == 1 and (rows >= 0).all() and (rows < N).all()
    o = np.empty((rows.size, d), np.float64)
    lse = np.empty(rows.size, np.float64)
    lib().oracle_fwd_rows(N, d, float(scale), int(causal), int(window),
                          _p(q), _p(k), _p(v),
                          rows.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                          rows.size, _p(o), _p(lse), int(nthreads))
    return o, lse


def probs_row(q, k, v, i: int, scale: float, causal: bool = False, window: int = 0):
    """The probability row P_i of ONE head."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    p = np.empty(N, np.float64)
    lib().oracle_probs_row(N, d, float(scale), int(causal), int(window),
                           _p(q), _p(k), _p(v), int(i), _p(p))
    return p


def bwd(q, k, v, dout, scale: float, causal: bool = False, window: int = 0,
        nthreads: int = 0):
    """dQ, dK, dV and D (D_i = sum_j P_ij dP_ij) for tensors [..., N, d]."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    assert q.shape == k.shape == v.shape == dout.shape
    N, d = q.shape[-2:]
    BH = int(np.prod(q.shape[:-2])) if q.ndim > 2 else 1
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    D = np.empty(q.shape[:-1], np.float64)
    lib().oracle_bwd(BH, N, d, float(scale), int(causal), int(window),
                     _p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv),
                     _p(D), int(nthreads))
    return dq, dk, dv, D


def online_fwd(q, k, v, bounds, form: int, scale: float, causal: bool = False,
               window: int = 0):
    """Block recurrence over the key partition ``bounds`` (form 1 or 2), ONE head."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    b = np.ascontiguousarray(bounds, dtype=np.int64)
    assert b[0] == 0 and b[-1] == N and (np.diff(b) > 0).all()
    o = np.empty_like(q)
    lse = np.empty(N, np.float64)
    lib().oracle_online_fwd(N, d, float(scale), int(causal), int(window),
                            _p(q), _p(k), _p(v),
                            b.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                            b.size - 1, int(form), _p(o), _p(lse))
    return o, lse


def _gqa_shapes(q, k):
    assert q.ndim == 4 and k.ndim == 4
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and Hkv >= 1 and H % Hkv == 0
    return B, H, Hkv, N, d


def fwd_gqa(q, k, v, scale: float, causal: bool = False, window: int = 0,
            nthreads: int = 0):
    """O and L for q [B, H, N, d] and shared k, v [B, Hkv, N, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Hkv, N, d = _gqa_shapes(q, k)
    assert v.shape == k.shape
    o = np.empty_like(q)
    lse = np.empty(q.shape[:-1], np.float64)
    lib().oracle_fwd_gqa(B, H, Hkv, N, d, float(scale), int(causal), int(window),
                         _p(q), _p(k), _p(v), _p(o), _p(lse), int(nthreads))
    return o, lse


def bwd_gqa(q, k, v, dout, scale: float, causal: bool = False, window: int = 0,
            nthreads: int = 0):
    """dQ [B, H, N, d], dK, dV [B, Hkv, N, d] (summed over each group) and D."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, Hkv, N, d = _gqa_shapes(q, k)
    assert v.shape == k.shape and dout.shape == q.shape
    dq = np.empty_like(q)
    dk, dv = np.empty_like(k), np.empty_like(k)
    D = np.empty(q.shape[:-1], np.float64)
    lib().oracle_bwd_gqa(B, H, Hkv, N, d, float(scale), int(causal), int(window),
                         _p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv), _p(D),
                         int(nthreads))
    return dq, dk, dv, D


def fwd_decode(q, k, v, scale: float, causal: bool = False, window: int = 0,
               nthreads: int = 0):
    """O and L for a block of Nq queries q [B, H, Nq, d] that are the last Nq
    positions of a sequence of Nk keys k, v [B, Hkv, Nk, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    assert q.ndim == 4 and k.ndim == 4 and v.shape == k.shape
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    assert k.shape == (B, Hkv, Nk, d) and H % Hkv == 0 and 1 <= Nq <= Nk
    o = np.empty_like(q)
    lse = np.empty(q.shape[:-1], np.float64)
    lib().oracle_fwd_decode(B, H, Hkv, Nq, Nk, d, float(scale), int(causal), int(window),
                            _p(q), _p(k), _p(v), _p(o), _p(lse), int(nthreads))
    return o, lse


# ---- dropout ----

def _u64(words):
    a = np.ascontiguousarray(words, dtype=np.uint64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))


def philox(width: int, rounds: int, counter, key) -> np.ndarray:
    """Philox-4x<width>-<rounds> of one 4-word counter and 2-word key (uint64 words)."""
    assert width in (32, 64) and rounds >= 1
    c, cp = _u64(counter)
    k, kp = _u64(key)
    assert c.shape == (4,) and k.shape == (2,)
    out, op = _u64(np.zeros(4))
    lib().oracle_philox(width, rounds, cp, kp, op)
    return out


def philox_constants(width: int) -> np.ndarray:
    """(M0, M1, W0, W1) of the width-bit Philox."""
    out, op = _u64(np.zeros(4))
    lib().oracle_philox_constants(width, op)
    return out


def dropout_threshold(p: float) -> int:
    """Integer threshold t = round(256 p); bytes below t are dropped."""
    return int(lib().oracle_dropout_threshold(float(p)))


def dropout_byte(seed: int, offset: int, bh: int, i: int, j: int) -> int:
    return int(lib().oracle_dropout_byte(seed, offset, bh, i, j))


def dropout_mask(seed: int, offset: int, p: float, bh: int, rows: int, cols: int,
                 i0: int = 0, j0: int = 0) -> np.ndarray:
    """Keep indicators Z (uint8 0/1) of query head bh, rows i0.., keys j0..."""
    z = np.empty((rows, cols), np.uint8)
    lib().oracle_dropout_mask(seed, offset, dropout_threshold(p), bh, i0, j0, rows, cols,
                              z.ctypes.data)
    return z


def fwd_dropout(q, k, v, scale: float, p: float, seed: int, offset: int = 0,
                causal: bool = False, window: int = 0, nthreads: int = 0, bh0: int = 0):
    """O (with dropout on P) and L for q [B, H, N, d], k, v [B, Hkv, N, d]; the
    query heads are heads bh0, bh0 + 1, ... of the generator's numbering."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Hkv, N, d = _gqa_shapes(q, k)
    assert v.shape == k.shape
    o = np.empty_like(q)
    lse = np.empty(q.shape[:-1], np.float64)
    lib().oracle_fwd_dropout(B, H, Hkv, N, d, float(scale), int(causal), int(window),
                             float(p), int(seed), int(offset), int(bh0), _p(q), _p(k),
                             _p(v), _p(o), _p(lse), int(nthreads))
    return o, lse


def bwd_dropout(q, k, v, dout, scale: float, p: float, seed: int, offset: int = 0,
                causal: bool = False, window: int = 0, nthreads: int = 0, bh0: int = 0):
    """dQ, dK, dV (summed over each group) and D of attention with dropout on P
    (head numbering as fwd_dropout)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, Hkv, N, d = _gqa_shapes(q, k)
    assert v.shape == k.shape and dout.shape == q.shape
    dq = np.empty_like(q)
    dk, dv = np.empty_like(k), np.empty_like(k)
    D = np.empty(q.shape[:-1], np.float64)
    lib().oracle_bwd_dropout(B, H, Hkv, N, d, float(scale), int(causal), int(window),
                             float(p), int(seed), int(offset), int(bh0), _p(q), _p(k),
                             _p(v), _p(dout), _p(dq), _p(dk), _p(dv), _p(D), int(nthreads))
    return dq, dk, dv, D

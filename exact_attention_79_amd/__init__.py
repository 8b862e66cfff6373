"""Exact attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/attn.h`` (``libattn.so``):
the functions below only check tensor metadata, allocate outputs with
PyTorch, and pass raw device pointers and the current HIP stream to the
library.  Every step of the computation runs in the library's HIP kernels.
There is no fallback: if ``libattn.so`` is missing, importing the binding
raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP, ATTN_ESCRATCH = 0, 1, 2, 3, 4
ATTN_OUT_BF16, ATTN_OUT_F32 = 0, 1
STAGE_FWD, STAGE_BWD_DQ, STAGE_BWD_DKDV, STAGE_FWD_FP8 = 0, 1, 2, 3

# Entry points declared in include/attn.h.
EXPORTS = ("attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_preprocess",
           "attn_bwd_dkdv", "attn_bwd_dq", "attn_fwd_fp8", "attn_decode_workspace_bytes",
           "attn_fwd_decode", "attn_fwd_fp8_blocks", "attn_fwd_dropout", "attn_bwd_dropout",
           "attn_status_str", "attn_kernel_name", "attn_bwd_noalloc",
           "attn_bwd_noalloc_scratch_bytes")


class AttnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("window", ctypes.c_int32), ("H_kv", ctypes.c_int32)]


class AttnDecodeDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("N_q", ctypes.c_int32), ("N_k", ctypes.c_int32), ("d", ctypes.c_int32),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("window", ctypes.c_int32)]


class AttnDropout(ctypes.Structure):
    _fields_ = [("p", ctypes.c_float), ("offset", ctypes.c_uint32),
                ("seed", ctypes.c_uint64)]


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python exact_attention_79_amd/build.py` "
            "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    dp = ctypes.POINTER(AttnDesc)
    L.attn_fwd.argtypes = [dp, vp, vp, vp, vp, i32, vp, vp]
    L.attn_fwd.restype = ctypes.c_int
    L.attn_bwd_workspace_bytes.argtypes = [dp]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_bwd.restype = ctypes.c_int
    L.attn_bwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attn_bwd_noalloc.restype = ctypes.c_int
    L.attn_bwd_noalloc_scratch_bytes.argtypes = [dp]
    L.attn_bwd_noalloc_scratch_bytes.restype = sz
    L.attn_bwd_preprocess.argtypes = [dp, vp, vp, vp, vp, sz, vp]
    L.attn_bwd_preprocess.restype = ctypes.c_int
    L.attn_bwd_dq.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    L.attn_bwd_dq.restype = ctypes.c_int
    L.attn_bwd_dkdv.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    L.attn_bwd_dkdv.restype = ctypes.c_int
    L.attn_fwd_fp8.argtypes = [dp, vp, vp, vp, f32, f32, f32, vp, i32, vp, vp]
    L.attn_fwd_fp8.restype = ctypes.c_int
    L.attn_fwd_fp8_blocks.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
    L.attn_fwd_fp8_blocks.restype = ctypes.c_int
    ddp = ctypes.POINTER(AttnDecodeDesc)
    L.attn_decode_workspace_bytes.argtypes = [ddp]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_fwd_decode.argtypes = [ddp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
    L.attn_fwd_decode.restype = ctypes.c_int
    drp = ctypes.POINTER(AttnDropout)
    L.attn_fwd_dropout.argtypes = [dp, drp, vp, vp, vp, vp, i32, vp, vp]
    L.attn_fwd_dropout.restype = ctypes.c_int
    L.attn_bwd_dropout.argtypes = [dp, drp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.attn_bwd_dropout.restype = ctypes.c_int
    L.attn_kernel_name.argtypes = [dp, i32, f32]
    L.attn_kernel_name.restype = ctypes.c_char_p
    L.attn_status_str.argtypes = [ctypes.c_int]
    L.attn_status_str.restype = ctypes.c_char_p
    return L


lib = _load()


def status_str(status: int) -> str:
    return lib.attn_status_str(int(status)).decode()


def kernel_name(stage: int, B: int, H: int, N: int, d: int, causal: bool = False,
                window: int = 0, H_kv: int = 0, dropout_p: float = 0.0) -> str:
    """Symbol of the main kernel that an entry point launches for this shape
    (stage: STAGE_FWD, STAGE_BWD_DQ, STAGE_BWD_DKDV or STAGE_FWD_FP8), as
    profilers list it; nothing is launched."""
    desc = make_desc(B, H, N, d, 1.0 / math.sqrt(d), causal, window, H_kv)
    name = lib.attn_kernel_name(ctypes.byref(desc), int(stage), float(dropout_p))
    if name is None:
        raise ValueError("invalid shape, stage or dropout probability")
    return name.decode()


def make_desc(B: int, H: int, N: int, d: int, scale: float, causal: bool,
              window: int, H_kv: int = 0) -> AttnDesc:
    return AttnDesc(int(B), int(H), int(N), int(d), float(scale), int(bool(causal)),
                    int(window), int(H_kv))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != ATTN_OK:
        raise AttnError(status, where)


def _check_qkv(q, k, v, dtypes):
    """q: [B, H, N, d]; k, v: [B, H_kv, N, d] with H a multiple of H_kv
    (shared key/value heads; H_kv = H is ordinary multi-head attention)."""
    for t in (q, k, v):
        if not t.is_cuda or t.dtype not in dtypes or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors of dtype "
                             f"{dtypes}")
        if t.dim() != 4:
            raise ValueError("q, k, v must be 4-d tensors [B, heads, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if (k.shape != (B, Hkv, N, d) or v.shape != k.shape or Hkv < 1 or H % Hkv):
        raise ValueError("q must be [B, H, N, d] and k, v [B, H_kv, N, d] with H a "
                         "multiple of H_kv")


def _fwd_prep(q, k, v, scale, causal, window, out_dtype, return_lse, out, lse):
    """Checks, outputs and descriptor of the bf16 forward."""
    _check_qkv(q, k, v, (torch.bfloat16,))
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    o = torch.empty_like(q, dtype=out_dtype) if out is None else out
    _check_like(q, out_dtype, out=o)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    _check_lse(lse, (B, H, N))
    desc = make_desc(B, H, N, d, scale, causal, window, k.shape[1])
    od = ATTN_OUT_F32 if out_dtype == torch.float32 else ATTN_OUT_BF16
    return desc, o, lse, od


def attn_fwd(q, k, v, scale: float | None = None, causal: bool = False,
             window: int = 0, out_dtype=torch.bfloat16, return_lse: bool = True,
             out=None, lse=None):
    """O (and the fp32 LSE) for bf16 q, k, v of shape [B, H, N, d]."""
    desc, o, lse, od = _fwd_prep(q, k, v, scale, causal, window, out_dtype, return_lse,
                                 out, lse)
    _check(lib.attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), od,
                        _ptr(lse), _stream()), "attn_fwd")
    return (o, lse) if return_lse else o


def make_dropout(p: float, seed: int, offset: int = 0) -> AttnDropout:
    """Dropout description: probability p, Philox key `seed`, counter word `offset`."""
    if not (0 <= seed < 2**64 and 0 <= offset < 2**32):
        raise ValueError("seed must fit in 64 bits and offset in 32 bits")
    return AttnDropout(float(p), int(offset), int(seed))


def attn_fwd_dropout(q, k, v, p: float, seed: int, offset: int = 0,
                     scale: float | None = None, causal: bool = False, window: int = 0,
                     out_dtype=torch.bfloat16, return_lse: bool = True, out=None, lse=None):
    """attn_fwd with dropout on P (keep bytes from Philox-4x32-10, see attn.h)."""
    desc, o, lse, od = _fwd_prep(q, k, v, scale, causal, window, out_dtype, return_lse,
                                 out, lse)
    drop = make_dropout(p, seed, offset)
    _check(lib.attn_fwd_dropout(ctypes.byref(desc), ctypes.byref(drop), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(o), od, _ptr(lse), _stream()),
           "attn_fwd_dropout")
    return (o, lse) if return_lse else o


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int, H_kv: int = 0,
                             causal: bool = False) -> int:
    """Workspace bytes of the backward (see include/attn.h; grouped-query
    backwards may need partial dK/dV space, which depends on H_kv and causal)."""
    desc = make_desc(B, H, N, d, 1.0, causal, 0, H_kv)
    return int(lib.attn_bwd_workspace_bytes(ctypes.byref(desc)))


def _bwd_prep(q, k, v, o, dout, lse, scale, causal, window, workspace, grads):
    """Checks, outputs, workspace and descriptor of the bf16 backward."""
    _check_qkv(q, k, v, (torch.bfloat16,))
    _check_like(q, torch.bfloat16, o=o, dout=dout)
    desc = _bwd_desc(q, k, scale, causal, window)
    nbytes = int(lib.attn_bwd_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), device=q.device, dtype=torch.uint8)
    if grads is None:
        grads = _new_grads(q, k)
    dq, dk, dv = grads
    _check_like(q, torch.float32, dq=dq)
    _check_like(k, torch.float32, dk=dk, dv=dv)
    _check_lse_ws(q, lse, workspace, desc)
    return desc, workspace, (dq, dk, dv)


def attn_bwd(q, k, v, o, dout, lse, scale: float | None = None,
             causal: bool = False, window: int = 0, workspace=None, grads=None):
    """dQ, dK, dV (fp32) for bf16 q, k, v, o, dout and the forward's fp32 lse."""
    desc, workspace, (dq, dk, dv) = _bwd_prep(q, k, v, o, dout, lse, scale, causal, window,
                                              workspace, grads)
    _check(lib.attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                        _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        _ptr(workspace), _ws_bytes(workspace), _stream()), "attn_bwd")
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, dout, lse, grads, scale: float | None = None,
                     causal: bool = False, window: int = 0):
    """attn_bwd without a workspace: the library's static device scratch holds
    D and L log2(e) (include/attn.h); the caller passes the fp32 gradient
    tensors (dq, dk, dv), so nothing is allocated."""
    _check_qkv(q, k, v, (torch.bfloat16,))
    _check_like(q, torch.bfloat16, o=o, dout=dout)
    dq, dk, dv = grads
    _check_like(q, torch.float32, dq=dq)
    _check_like(k, torch.float32, dk=dk, dv=dv)
    B, H, N, _ = q.shape
    _check_lse(lse, (B, H, N))
    desc = _bwd_desc(q, k, scale, causal, window)
    _check(lib.attn_bwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                _stream()), "attn_bwd_noalloc")
    return dq, dk, dv


def attn_bwd_dropout(q, k, v, o, dout, lse, p: float, seed: int, offset: int = 0,
                     scale: float | None = None, causal: bool = False, window: int = 0,
                     workspace=None, grads=None):
    """attn_bwd of attn_fwd_dropout (same p, seed and offset as that forward)."""
    desc, workspace, (dq, dk, dv) = _bwd_prep(q, k, v, o, dout, lse, scale, causal, window,
                                              workspace, grads)
    drop = make_dropout(p, seed, offset)
    _check(lib.attn_bwd_dropout(ctypes.byref(desc), ctypes.byref(drop), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(workspace), _ws_bytes(workspace), _stream()),
           "attn_bwd_dropout")
    return dq, dk, dv


def _bwd_desc(q, k, scale, causal, window):
    """Descriptor from q's shape and, when given, the key/value head count of k."""
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    return make_desc(B, H, N, d, scale, causal, window, 0 if k is None else k.shape[1])


def _new_grads(q, k):
    dq = torch.empty(q.shape, device=q.device, dtype=torch.float32)
    dk, dv = (torch.empty(k.shape, device=q.device, dtype=torch.float32) for _ in range(2))
    return dq, dk, dv


def _check_like(ref, dtype, **tensors):
    for name, t in tensors.items():
        if (not t.is_cuda or t.shape != ref.shape or t.dtype != dtype
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {dtype} device tensor "
                             f"of shape {tuple(ref.shape)}")


def _check_lse(lse, shape):
    """lse, when given, must be a contiguous fp32 device tensor of `shape`
    (the kernels write every element of it)."""
    if lse is not None and (not lse.is_cuda or lse.dtype != torch.float32
                            or tuple(lse.shape) != tuple(shape) or not lse.is_contiguous()):
        dims = ", ".join(str(x) for x in shape)
        raise ValueError(f"lse must be a contiguous fp32 device tensor of shape [{dims}]")


def _check_lse_ws(q, lse, workspace, desc):
    B, H, N, _ = q.shape
    _check_lse(lse, (B, H, N))
    need = int(lib.attn_bwd_workspace_bytes(ctypes.byref(desc)))
    if workspace.numel() * workspace.element_size() < need or not workspace.is_cuda:
        raise ValueError(f"workspace must be a device tensor of >= {need} bytes")


def _ws_bytes(workspace):
    return workspace.numel() * workspace.element_size()


def attn_bwd_preprocess(o, dout, lse, workspace, scale=None, causal=False, window=0):
    """Fills the workspace only: D = rowsum(dO * O) and L log2(e)."""
    _check_like(o, torch.bfloat16, o=o, dout=dout)
    desc = _bwd_desc(o, None, scale, causal, window)
    _check_lse_ws(o, lse, workspace, desc)
    _check(lib.attn_bwd_preprocess(ctypes.byref(desc), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(workspace), _ws_bytes(workspace), _stream()),
           "attn_bwd_preprocess")


def attn_bwd_dq(q, k, v, o, dout, lse, workspace, dq, scale=None, causal=False,
                window=0):
    """First backward stage: dQ (fp32); also fills the workspace (D, L log2(e))."""
    _check_qkv(q, k, v, (torch.bfloat16,))
    _check_like(q, torch.bfloat16, o=o, dout=dout)
    _check_like(q, torch.float32, dq=dq)
    desc = _bwd_desc(q, k, scale, causal, window)
    _check_lse_ws(q, lse, workspace, desc)
    _check(lib.attn_bwd_dq(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                           _ptr(dout), _ptr(lse), _ptr(workspace), _ws_bytes(workspace),
                           _ptr(dq), _stream()), "attn_bwd_dq")


def attn_bwd_dkdv(q, k, v, dout, workspace, dk, dv, scale=None, causal=False,
                  window=0):
    """Second backward stage: dK and dV (fp32), from the workspace that
    attn_bwd_dq (or attn_bwd_preprocess) filled."""
    _check_qkv(q, k, v, (torch.bfloat16,))
    _check_like(q, torch.bfloat16, dout=dout)
    _check_like(k, torch.float32, dk=dk, dv=dv)
    desc = _bwd_desc(q, k, scale, causal, window)
    _check_lse_ws(q, None, workspace, desc)
    _check(lib.attn_bwd_dkdv(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                             _ptr(workspace), _ws_bytes(workspace), _ptr(dk), _ptr(dv),
                             _stream()), "attn_bwd_dkdv")


def attn_bwd_stages(q, k, v, o, dout, lse, scale: float | None = None,
                    causal: bool = False, window: int = 0, workspace=None,
                    grads=None, preprocess: bool = False):
    """The result of attn_bwd, issued stage by stage: attn_bwd_dq, then
    attn_bwd_dkdv (exactly what attn_bwd enqueues).  With preprocess=True:
    attn_bwd_preprocess, attn_bwd_dkdv, then attn_bwd_dq, so that dK and dV
    come from the workspace the preprocess filled."""
    desc = _bwd_desc(q, k, scale, causal, window)
    if workspace is None:
        nbytes = int(lib.attn_bwd_workspace_bytes(ctypes.byref(desc)))
        workspace = torch.empty(max(nbytes, 1), device=q.device, dtype=torch.uint8)
    if grads is None:
        grads = _new_grads(q, k)
    dq, dk, dv = grads
    kw = dict(scale=scale, causal=causal, window=window)
    if preprocess:
        attn_bwd_preprocess(o, dout, lse, workspace, **kw)
        attn_bwd_dkdv(q, k, v, dout, workspace, dk, dv, **kw)
        attn_bwd_dq(q, k, v, o, dout, lse, workspace, dq, **kw)
    else:
        attn_bwd_dq(q, k, v, o, dout, lse, workspace, dq, **kw)
        attn_bwd_dkdv(q, k, v, dout, workspace, dk, dv, **kw)
    return dq, dk, dv


def attn_fwd_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float,
                 scale: float | None = None, causal: bool = False, window: int = 0,
                 out_dtype=torch.bfloat16, return_lse: bool = True, out=None, lse=None):
    """O (and LSE) for e4m3 codes (uint8 or float8_e4m3fn) q8 [B, H, N, d] and
    k8, v8 [B, H_kv, N, d]; the inputs are code * descale."""
    _check_qkv(q8, k8, v8, (torch.uint8, torch.float8_e4m3fn))
    B, H, N, d = q8.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    o = torch.empty(q8.shape, device=q8.device, dtype=out_dtype) if out is None else out
    _check_like(q8, out_dtype, out=o)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), device=q8.device, dtype=torch.float32)
    _check_lse(lse, (B, H, N))
    desc = make_desc(B, H, N, d, scale, causal, window, k8.shape[1])
    od = ATTN_OUT_F32 if out_dtype == torch.float32 else ATTN_OUT_BF16
    _check(lib.attn_fwd_fp8(ctypes.byref(desc), _ptr(q8), _ptr(k8), _ptr(v8),
                            float(q_descale), float(k_descale), float(v_descale),
                            _ptr(o), od, _ptr(lse), _stream()), "attn_fwd_fp8")
    return (o, lse) if return_lse else o


def make_decode_desc(B: int, H: int, H_kv: int, N_q: int, N_k: int, d: int, scale: float,
                     causal: bool, window: int) -> AttnDecodeDesc:
    return AttnDecodeDesc(int(B), int(H), int(H_kv), int(N_q), int(N_k), int(d),
                          float(scale), int(bool(causal)), int(window))


def attn_decode_workspace_bytes(B: int, H: int, H_kv: int, N_q: int, N_k: int, d: int,
                                causal: bool = False, window: int = 0) -> int:
    desc = make_decode_desc(B, H, H_kv, N_q, N_k, d, 1.0, causal, window)
    return int(lib.attn_decode_workspace_bytes(ctypes.byref(desc)))


def attn_fwd_decode(q, k, v, scale: float | None = None, causal: bool = False,
                    window: int = 0, out_dtype=torch.bfloat16, return_lse: bool = True,
                    out=None, lse=None, workspace=None):
    """O (and LSE) for a block of N_q queries q [B, H, N_q, d] that are the last
    N_q positions of the N_k keys k, v [B, H_kv, N_k, d] (bf16)."""
    for t in (q, k, v):
        if (not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous()
                or t.dim() != 4):
            raise ValueError("q, k, v must be contiguous 4-d bf16 device tensors")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != k.shape or H % Hkv or Nq > Nk:
        raise ValueError("q must be [B, H, N_q, d], k and v [B, H_kv, N_k, d] with H a "
                         "multiple of H_kv and N_q <= N_k")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    o = torch.empty(q.shape, device=q.device, dtype=out_dtype) if out is None else out
    _check_like(q, out_dtype, out=o)
    if return_lse and lse is None:
        lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    _check_lse(lse, (B, H, Nq))
    desc = make_decode_desc(B, H, Hkv, Nq, Nk, d, scale, causal, window)
    need = int(lib.attn_decode_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    if not workspace.is_cuda or _ws_bytes(workspace) < need:
        raise ValueError(f"workspace must be a device tensor of >= {need} bytes")
    od = ATTN_OUT_F32 if out_dtype == torch.float32 else ATTN_OUT_BF16
    _check(lib.attn_fwd_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), od,
                               _ptr(lse), _ptr(workspace), _ws_bytes(workspace),
                               _stream()), "attn_fwd_decode")
    return (o, lse) if return_lse else o


def attn_fwd_fp8_blocks(q8, k8, v8, q_descales, k_descales, v_descales,
                        scale: float | None = None, causal: bool = False, window: int = 0,
                        out_dtype=torch.bfloat16, return_lse: bool = True, out=None,
                        lse=None):
    """fp8 forward with one descale per block: q_descales fp32 [B, H, ceil(N/128)],
    k_descales and v_descales fp32 [B, H_kv, ceil(N/64)] (device tensors)."""
    _check_qkv(q8, k8, v8, (torch.uint8, torch.float8_e4m3fn))
    B, H, N, d = q8.shape
    Hkv = k8.shape[1]
    shapes = {"q_descales": (q_descales, (B, H, (N + 127) // 128)),
              "k_descales": (k_descales, (B, Hkv, (N + 63) // 64)),
              "v_descales": (v_descales, (B, Hkv, (N + 63) // 64))}
    for name, (t, shp) in shapes.items():
        if (not t.is_cuda or t.dtype != torch.float32 or tuple(t.shape) != shp
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 device tensor {shp}")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    o = torch.empty(q8.shape, device=q8.device, dtype=out_dtype) if out is None else out
    _check_like(q8, out_dtype, out=o)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), device=q8.device, dtype=torch.float32)
    _check_lse(lse, (B, H, N))
    desc = make_desc(B, H, N, d, scale, causal, window, Hkv)
    od = ATTN_OUT_F32 if out_dtype == torch.float32 else ATTN_OUT_BF16
    _check(lib.attn_fwd_fp8_blocks(ctypes.byref(desc), _ptr(q8), _ptr(k8), _ptr(v8),
                                   _ptr(q_descales), _ptr(k_descales), _ptr(v_descales),
                                   _ptr(o), od, _ptr(lse), _stream()), "attn_fwd_fp8_blocks")
    return (o, lse) if return_lse else o

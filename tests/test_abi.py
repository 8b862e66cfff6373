"""Host-side checks of the C ABI: the library loads, exports every entry point
that include/attn.h declares, and rejects bad arguments before launching
anything (these paths make no HIP call, so they run without a GPU)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def ea():
    import exact_attention_79_amd as ea
    return ea


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_preprocess",
         "attn_bwd_dkdv", "attn_bwd_dq", "attn_fwd_fp8", "attn_decode_workspace_bytes",
         "attn_fwd_decode", "attn_fwd_fp8_blocks", "attn_fwd_dropout", "attn_bwd_dropout",
         "attn_status_str", "attn_kernel_name", "attn_bwd_noalloc",
         "attn_bwd_noalloc_scratch_bytes"])


def test_library_exports_every_declared_symbol(ea):
    for name in declared_functions():
        assert hasattr(ea.lib, name), name
    assert set(ea.EXPORTS) == set(declared_functions())


def test_status_strings(ea):
    for s in range(5):
        assert ea.status_str(s) and ea.status_str(s) != "unknown status"
    assert ea.status_str(99) == "unknown status"


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def call_fwd(ea, desc, q=FAKE, k=FAKE, v=FAKE, o=FAKE, od=0, lse=None):
    vp = ctypes.c_void_p
    return ea.lib.attn_fwd(ctypes.byref(desc), vp(q), vp(k), vp(v), vp(o), od,
                           vp(lse) if lse else None, None)


@pytest.mark.parametrize("field,value,expect", [
    ("B", 0, 1), ("H", -1, 1), ("N", 0, 1), ("window", -1, 1), ("causal", 2, 1),
    ("scale", 0.0, 1), ("scale", -1.0, 1), ("scale", math.inf, 1), ("scale", math.nan, 1),
    ("d", 32, 2), ("d", 96, 2), ("d", 256, 2),
])
def test_fwd_rejects_bad_descriptors(ea, field, value, expect):
    desc = ea.make_desc(1, 1, 16, 64, 0.125, False, 0)
    setattr(desc, field, value)
    assert call_fwd(ea, desc) == expect


@pytest.mark.parametrize("H,H_kv,expect", [(4, 3, 1), (4, -1, 1), (6, 4, 1), (4, 0, 0),
                                            (4, 4, 0), (4, 2, 0), (4, 1, 0)])
def test_shared_kv_head_counts(ea, H, H_kv, expect):
    """H_kv must be 0 or a divisor of H: an invalid descriptor has no
    workspace size (0) and is refused by every entry point."""
    desc = ea.make_desc(1, H, 16, 64, 0.125, False, 0, H_kv)
    ws = ea.lib.attn_bwd_workspace_bytes(ctypes.byref(desc))
    assert (ws == 0) == (expect == 1)
    if expect == 1:
        assert call_fwd(ea, desc) == ea.ATTN_EINVAL


def test_fwd_rejects_bad_pointers_and_dtype(ea):
    desc = ea.make_desc(1, 1, 16, 64, 0.125, False, 0)
    assert call_fwd(ea, desc, q=0) == ea.ATTN_EINVAL
    assert call_fwd(ea, desc, o=0) == ea.ATTN_EINVAL
    assert call_fwd(ea, desc, k=FAKE + 8) == ea.ATTN_EINVAL
    assert call_fwd(ea, desc, lse=FAKE + 4) == ea.ATTN_EINVAL
    assert call_fwd(ea, desc, od=7) == ea.ATTN_EINVAL
    big = ea.make_desc(1 << 10, 1 << 10, 1 << 10, 128, 0.1, False, 0)
    assert call_fwd(ea, big) == ea.ATTN_EUNSUPPORTED


def test_bwd_workspace_and_rejections(ea):
    desc = ea.make_desc(2, 3, 100, 128, 0.1, True, 0)
    ws = ea.lib.attn_bwd_workspace_bytes(ctypes.byref(desc))
    assert ws >= 2 * (2 * 3 * 100 * 4) and ws % 256 == 0  # D and L log2(e)
    bad = ea.make_desc(2, 3, 100, 80, 0.1, True, 0)
    assert ea.lib.attn_bwd_workspace_bytes(ctypes.byref(bad)) == 0
    vp = ctypes.c_void_p
    args = [vp(FAKE)] * 10
    assert ea.lib.attn_bwd(ctypes.byref(desc), *args, ws - 1, None) == ea.ATTN_EINVAL
    args[5] = None  # lse
    assert ea.lib.attn_bwd(ctypes.byref(desc), *args, ws, None) == ea.ATTN_EINVAL
    assert ea.lib.attn_bwd(ctypes.byref(bad), *([vp(FAKE)] * 10), ws, None) == \
        ea.ATTN_EUNSUPPORTED


def split_of(B, H, H_kv, N, d, causal):
    """The documented share count of the grouped dK/dV walk (include/attn.h)."""
    G, grid = H // H_kv, B * H_kv * ((N + 127) // 128)
    want = 256 * (2 if d == 64 else 1) * (2 if causal else 1)
    if G <= 1 or grid >= want:
        return 1
    return next((s for s in range(2, G) if G % s == 0 and grid * s >= want), G)


@pytest.mark.parametrize("B,H,H_kv,N,d,causal,S", [
    (4, 16, 16, 2048, 128, True, 1), (4, 16, 4, 2048, 128, False, 1),
    (4, 16, 4, 2048, 128, True, 2), (4, 16, 4, 2048, 64, True, 4),
    (4, 16, 4, 2048, 64, False, 2), (1, 8, 1, 2048, 64, False, 8),
    (2, 6, 3, 100, 64, True, 2), (8, 32, 8, 4096, 128, True, 1),
    (4, 16, 4, 4096, 128, True, 1), (2, 12, 2, 1024, 128, True, 6)])
def test_bwd_workspace_holds_the_split_partials(ea, B, H, H_kv, N, d, causal, S):
    """Grouped-query backwards whose dK/dV grid would be small split each
    group over S workgroups and keep S partial dK and dV arrays in the
    workspace, after the D and L log2(e) arrays."""
    assert split_of(B, H, H_kv, N, d, causal) == S
    pad = lambda x: (x + 255) // 256 * 256
    want = 2 * pad(B * H * N * 4)
    if S > 1:
        want += 2 * pad(S * B * H_kv * N * d * 4)
    assert ea.attn_bwd_workspace_bytes(B, H, N, d, H_kv, causal) == want


def test_bwd_stages_reject_bad_arguments(ea):
    desc = ea.make_desc(1, 2, 64, 64, 0.1, False, 0)
    ws = ea.lib.attn_bwd_workspace_bytes(ctypes.byref(desc))
    vp = ctypes.c_void_p
    f = vp(FAKE)
    assert ea.lib.attn_bwd_preprocess(ctypes.byref(desc), f, None, f, f, ws, None) == 1
    assert ea.lib.attn_bwd_preprocess(ctypes.byref(desc), f, f, None, f, ws, None) == 1
    assert ea.lib.attn_bwd_preprocess(ctypes.byref(desc), f, f, f, f, ws - 1, None) == 1
    assert ea.lib.attn_bwd_dkdv(ctypes.byref(desc), f, f, f, f, f, ws, f, vp(FAKE + 4),
                                None) == 1
    assert ea.lib.attn_bwd_dkdv(ctypes.byref(desc), f, f, f, f, None, ws, f, f, None) == 1
    assert ea.lib.attn_bwd_dq(ctypes.byref(desc), f, f, None, f, f, f, f, ws, f, None) == 1
    assert ea.lib.attn_bwd_dq(ctypes.byref(desc), f, f, f, None, f, f, f, ws, f, None) == 1
    assert ea.lib.attn_bwd_dq(ctypes.byref(desc), f, f, f, f, f, f, f, ws - 1, f,
                              None) == 1
    bad = ea.make_desc(1, 2, 64, 64, -0.1, False, 0)
    assert ea.lib.attn_bwd_dq(ctypes.byref(bad), f, f, f, f, f, f, f, ws, f, None) == 1


def test_fp8_rejects_bad_descales(ea):
    desc = ea.make_desc(1, 1, 16, 128, 0.1, False, 0)
    vp = ctypes.c_void_p
    for qs, ks, vs in ((0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, math.nan)):
        assert ea.lib.attn_fwd_fp8(ctypes.byref(desc), vp(FAKE), vp(FAKE), vp(FAKE),
                                   qs, ks, vs, vp(FAKE), 0, None, None) == ea.ATTN_EINVAL


@pytest.mark.parametrize("p,expect", [(-0.1, 1), (math.nan, 1), (math.inf, 1),
                                      (255.5 / 256, 1), (0.999, 1)])
def test_dropout_rejects_bad_probabilities(ea, p, expect):
    """p must be finite, >= 0, with round(256 p) <= 255; checked before any launch."""
    desc = ea.make_desc(1, 2, 64, 64, 0.1, False, 0)
    ws = ea.lib.attn_bwd_workspace_bytes(ctypes.byref(desc))
    vp = ctypes.c_void_p
    f = vp(FAKE)
    drop = ea.AttnDropout(p, 0, 1)
    assert ea.lib.attn_fwd_dropout(ctypes.byref(desc), ctypes.byref(drop), f, f, f, f, 0,
                                   None, None) == expect
    assert ea.lib.attn_bwd_dropout(ctypes.byref(desc), ctypes.byref(drop), *([f] * 10), ws,
                                   None) == expect


def test_dropout_rejects_null_description_and_bad_arguments(ea):
    desc = ea.make_desc(1, 2, 64, 64, 0.1, False, 0)
    ws = ea.lib.attn_bwd_workspace_bytes(ctypes.byref(desc))
    vp = ctypes.c_void_p
    f = vp(FAKE)
    drop = ea.AttnDropout(0.1, 0, 1)
    assert ea.lib.attn_fwd_dropout(ctypes.byref(desc), None, f, f, f, f, 0, None, None) == 1
    assert ea.lib.attn_bwd_dropout(ctypes.byref(desc), None, *([f] * 10), ws, None) == 1
    assert ea.lib.attn_fwd_dropout(ctypes.byref(desc), ctypes.byref(drop), f, None, f, f, 0,
                                   None, None) == 1
    assert ea.lib.attn_fwd_dropout(ctypes.byref(desc), ctypes.byref(drop), f, f, f, f, 5,
                                   None, None) == 1
    assert ea.lib.attn_bwd_dropout(ctypes.byref(desc), ctypes.byref(drop), *([f] * 10),
                                   ws - 1, None) == 1
    bad = ea.make_desc(1, 2, 64, 80, 0.1, False, 0)
    assert ea.lib.attn_fwd_dropout(ctypes.byref(bad), ctypes.byref(drop), f, f, f, f, 0,
                                   None, None) == 2
    assert ctypes.sizeof(ea.AttnDropout) == 16
    with pytest.raises(ValueError):
        ea.make_dropout(0.1, -1)


def test_binding_refuses_host_tensors(ea):
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.attn_fwd(q, q, q)


@pytest.mark.parametrize("field,value,expect", [
    ("N_q", 0, 1), ("N_q", 100, 1), ("N_k", 0, 1), ("H_kv", 3, 1), ("H_kv", -1, 1),
    ("window", -2, 1), ("scale", 0.0, 1), ("d", 96, 2), ("causal", 3, 1),
])
def test_decode_rejects_bad_descriptors(ea, field, value, expect):
    desc = ea.make_decode_desc(1, 4, 2, 4, 64, 64, 0.125, True, 0)
    assert ea.lib.attn_decode_workspace_bytes(ctypes.byref(desc)) > 0
    setattr(desc, field, value)
    assert ea.lib.attn_decode_workspace_bytes(ctypes.byref(desc)) == 0
    vp = ctypes.c_void_p
    f = vp(FAKE)
    assert ea.lib.attn_fwd_decode(ctypes.byref(desc), f, f, f, f, 0, None, f, 1 << 30,
                                  None) == expect


def test_decode_rejects_small_workspace_and_null_pointers(ea):
    desc = ea.make_decode_desc(2, 8, 2, 1, 5000, 128, 0.1, False, 0)
    ws = ea.lib.attn_decode_workspace_bytes(ctypes.byref(desc))
    assert ws > 0 and ws % 256 == 0
    vp = ctypes.c_void_p
    f = vp(FAKE)
    assert ea.lib.attn_fwd_decode(ctypes.byref(desc), f, f, f, f, 0, None, f, ws - 1,
                                  None) == ea.ATTN_EINVAL
    assert ea.lib.attn_fwd_decode(ctypes.byref(desc), f, None, f, f, 0, None, f, ws,
                                  None) == ea.ATTN_EINVAL
    assert ea.lib.attn_fwd_decode(ctypes.byref(desc), f, f, f, f, 5, None, f, ws,
                                  None) == ea.ATTN_EINVAL


@pytest.mark.parametrize("stage,B,H,N,d,causal,p,expect", [
    (0, 4, 16, 2048, 128, False, 0.0, "attn::fwd_pp_kernel<128, 4, 32>"),
    (0, 4, 16, 2048, 64, True, 0.0, "attn::fwd_pp_kernel<64, 4, 64>"),
    (0, 1, 1, 256, 64, False, 0.0, "attn::fwd_bf16_kernel<64, 4, 64, false>"),
    (0, 4, 16, 2048, 128, False, 0.1, "attn::fwd_bf16_kernel<128, 4, 32, true>"),
    (1, 4, 16, 2048, 128, True, 0.0, "attn::bwd_dq_pp_kernel<128, 4>"),
    (1, 4, 16, 2048, 64, True, 0.0, "attn::bwd_dq_kernel<64, 4, 64, false>"),
    (1, 4, 16, 2048, 64, True, 0.1, "attn::bwd_dq_kernel<64, 4, 64, true>"),
    (2, 4, 16, 2048, 128, False, 0.0, "attn::bwd_dkdv_quad_kernel<128>"),
    (2, 4, 16, 2048, 64, False, 0.0, "attn::bwd_dkdv_pp_kernel<64, 4>"),
    (2, 4, 16, 2048, 64, True, 0.0, "attn::bwd_dkdv_kernel<64, 4, 32, false>"),
    (2, 4, 16, 2048, 128, True, 0.1, "attn::bwd_dkdv_kernel<128, 4, 32, true>"),
    (3, 2, 32, 8192, 128, False, 0.0, "attn::fwd_fp8_pp_kernel<128, 4, 32, false>"),
    (3, 2, 32, 8192, 64, False, 0.0, "attn::fwd_fp8_pp_kernel<64, 4, 64, false>"),
    (3, 1, 1, 256, 128, True, 0.0, "attn::fwd_fp8_pp_kernel<128, 4, 32, false>"),
])
def test_kernel_name_follows_the_dispatch(ea, stage, B, H, N, d, causal, p, expect):
    """The name query walks the same dispatch as the launch, without launching."""
    assert ea.kernel_name(stage, B, H, N, d, causal, dropout_p=p) == expect


def test_kernel_name_rejects_invalid_queries(ea):
    with pytest.raises(ValueError):
        ea.kernel_name(0, 1, 1, 64, 96)             # unsupported head dim
    with pytest.raises(ValueError):
        ea.kernel_name(7, 1, 1, 64, 64)             # no such stage
    with pytest.raises(ValueError):
        ea.kernel_name(3, 1, 1, 64, 128, dropout_p=0.1)  # fp8 has no dropout
    with pytest.raises(ValueError):
        ea.kernel_name(0, 1, 1, 64, 64, dropout_p=2.0)


class _FakeDeviceTensor:
    """Metadata-only stand-in for a device tensor (no GPU needed)."""

    def __init__(self, shape, dtype, contiguous=True):
        self.shape, self.dtype, self._c, self.is_cuda = tuple(shape), dtype, contiguous, True

    def is_contiguous(self):
        return self._c


def test_lse_check_shared_by_every_forward(ea):
    """Every forward entry (bf16, fp8, fp8 blocks, decode, and the backward's
    lse argument) goes through one lse check: shape, dtype and layout."""
    import inspect
    import torch
    ok = _FakeDeviceTensor((2, 3, 100), torch.float32)
    ea._check_lse(ok, (2, 3, 100))
    ea._check_lse(None, (2, 3, 100))
    for bad in (_FakeDeviceTensor((2, 3, 99), torch.float32),
                _FakeDeviceTensor((2, 3, 100), torch.bfloat16),
                _FakeDeviceTensor((2, 3, 100), torch.float32, contiguous=False),
                _FakeDeviceTensor((6, 100), torch.float32)):
        with pytest.raises(ValueError):
            ea._check_lse(bad, (2, 3, 100))
    for fn in (ea._fwd_prep, ea.attn_fwd_fp8, ea.attn_fwd_fp8_blocks, ea.attn_fwd_decode,
               ea._check_lse_ws):
        assert "_check_lse(lse" in inspect.getsource(fn), fn.__name__


def test_noalloc_backward_rejects_before_launching(ea):
    """The no-allocation backward checks its arguments like attn_bwd and
    refuses problems whose D and L log2(e) arrays exceed its static scratch
    (ATTN_ESCRATCH), all before any HIP call."""
    vp = ctypes.c_void_p
    f = vp(FAKE)
    limit = 16 << 20
    ok = ea.make_desc(4, 16, 4096, 128, 0.1, True, 0)
    need = ea.lib.attn_bwd_noalloc_scratch_bytes(ctypes.byref(ok))
    assert need == 2 * 4 * 16 * 4096 * 4 and need <= limit
    big = ea.make_desc(1, 64, 65536, 64, 0.1, True, 0)  # 2^22 rows: 32 MiB
    assert ea.lib.attn_bwd_noalloc_scratch_bytes(ctypes.byref(big)) > limit
    assert ea.lib.attn_bwd_noalloc(ctypes.byref(big), *([f] * 9), None) == ea.ATTN_ESCRATCH
    assert ea.lib.attn_bwd_noalloc(ctypes.byref(ok), f, f, f, f, f, None, f, f, f,
                                   None) == ea.ATTN_EINVAL
    assert ea.lib.attn_bwd_noalloc(ctypes.byref(ok), f, f, f, f, f, f, f, f, vp(FAKE + 4),
                                   None) == ea.ATTN_EINVAL
    bad = ea.make_desc(1, 2, 64, 80, 0.1, False, 0)
    assert ea.lib.attn_bwd_noalloc_scratch_bytes(ctypes.byref(bad)) == 0
    assert ea.lib.attn_bwd_noalloc(ctypes.byref(bad), *([f] * 9), None) == \
        ea.ATTN_EUNSUPPORTED

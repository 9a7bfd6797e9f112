"""The C-ABI library loads without a GPU, exports every symbol include/mla.h
declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest

from mla_latent_kv_04_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    for name in _declared():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings(lib):
    for code, name in [(0, "MLA_OK"), (1, "MLA_ERR_INVALID_ARG"), (2, "MLA_ERR_MISALIGNED"),
                       (3, "MLA_ERR_UNSUPPORTED"), (4, "MLA_ERR_WORKSPACE"), (5, "MLA_ERR_HIP")]:
        assert lib.mla_status_string(code).decode() == name
    assert lib.mla_status_string(99).decode() == "MLA_ERR_UNKNOWN"


def _params(**kw):
    p = _lib.DecodeParams()
    p.batch, p.s_q, p.num_heads, p.page_size, p.max_blocks_per_seq = 2, 1, 128, 64, 4
    p.num_splits, p.num_pages, p.scale, p.reserved = 8, 8, 0.0721687836, 0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


# Fake device addresses: validation rejects the call before anything dereferences them.
A = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)


def _paged(lib, p, ptrs=None, ws=A, ws_bytes=1 << 30):
    q, r, kv, bt, sl, ol, lse = ptrs or (A, A, A, A, A, A, None)
    return lib.mla_decode_paged(q, r, kv, bt, sl, ol, lse, ctypes.byref(p), ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("s_q", 257, _lib.MLA_ERR_UNSUPPORTED), ("s_q", 0, _lib.MLA_ERR_UNSUPPORTED),
    ("num_heads", 64, _lib.MLA_ERR_UNSUPPORTED), ("page_size", 16, _lib.MLA_ERR_UNSUPPORTED),
    ("batch", -1, _lib.MLA_ERR_INVALID_ARG), ("max_blocks_per_seq", 0, _lib.MLA_ERR_INVALID_ARG),
    ("num_pages", 0, _lib.MLA_ERR_INVALID_ARG), ("scale", 0.0, _lib.MLA_ERR_INVALID_ARG),
    ("scale", float("nan"), _lib.MLA_ERR_INVALID_ARG), ("num_splits", -2, _lib.MLA_ERR_INVALID_ARG),
    ("reserved", 1, _lib.MLA_ERR_INVALID_ARG),
])
def test_bad_params_rejected(lib, field, value, status):
    assert _paged(lib, _params(**{field: value})) == status
    assert lib.mla_last_error().decode() != ""


def test_page_sum_overflow_rejected(lib):
    """The decode sums 32-token tiles per (sequence, query) unit in 32-bit integers; a unit
    has at most two tiles per block-table entry, so 2 * batch * s_q * max_blocks_per_seq
    must stay below 2^31."""
    over = _params(batch=4096, s_q=2, max_blocks_per_seq=1 << 17, num_splits=8)     # exactly 2^31 tiles
    assert _paged(lib, over) == _lib.MLA_ERR_INVALID_ARG
    assert "2^31" in lib.mla_last_error().decode()
    assert lib.mla_decode_workspace_size(ctypes.byref(over), 0) == 0
    st = lib.mla_decode(A, A, A, A, A, A, A, A, None, ctypes.byref(over), A, 1 << 40, None)
    assert st == _lib.MLA_ERR_INVALID_ARG
    st = lib.mla_decode_paged_mxfp8(A, A, A, A, A, A, None, ctypes.byref(over), A, 1 << 40, None)
    assert st == _lib.MLA_ERR_INVALID_ARG
    # the cost line of the split adds 6 per unit and a range may start one range (at most
    # 2^16) past its end: 8192 * (2 * 131064 + 6) + 65536 fits, 131065 does not
    assert _paged(lib, _params(batch=4096, s_q=2, max_blocks_per_seq=131065, num_splits=8)) == \
        _lib.MLA_ERR_INVALID_ARG
    fits = _params(batch=4096, s_q=2, max_blocks_per_seq=131064, num_splits=8)
    assert lib.mla_decode_workspace_size(ctypes.byref(fits), 0) > 0


def test_null_params_and_pointers(lib):
    assert lib.mla_decode_paged(A, A, A, A, A, A, None, None, A, 1 << 30, None) == _lib.MLA_ERR_INVALID_ARG
    assert _paged(lib, _params(), (A, None, A, A, A, A, None)) == _lib.MLA_ERR_INVALID_ARG


@pytest.mark.parametrize("which", range(6))
def test_misaligned_tensors(lib, which):
    ptrs = [A, A, A, A, A, A, None]
    ptrs[which] = MIS if which != 4 else ctypes.c_void_p(0x10002)
    assert _paged(lib, _params(), tuple(ptrs)) == _lib.MLA_ERR_MISALIGNED


def test_workspace_checks(lib):
    p = _params()
    need = lib.mla_decode_workspace_size(ctypes.byref(p), 0)
    # cum [B*s_q+1] int32, partial lse [2W,128] fp32, partial O [2W,128,512] bf16 (each 256-B aligned)
    W = p.num_splits
    assert need == 256 + 2 * W * 128 * 4 + 2 * W * 128 * 512 * 2
    fused = lib.mla_decode_workspace_size(ctypes.byref(p), 1)
    assert fused == need + 2 * (2 * 128 * 512 * 2)
    assert _paged(lib, p, ws=A, ws_bytes=need - 1) == _lib.MLA_ERR_WORKSPACE
    assert _paged(lib, p, ws=None, ws_bytes=need) == _lib.MLA_ERR_WORKSPACE
    assert lib.mla_decode_workspace_size(ctypes.byref(_params(s_q=300)), 0) == 0
    assert lib.mla_decode_workspace_size(ctypes.byref(_params(s_q=256)), 0) > 0


def test_empty_batch_is_a_noop(lib):
    assert _paged(lib, _params(batch=0), (None,) * 6 + (None,), ws=None, ws_bytes=0) == _lib.MLA_OK
    assert lib.mla_absorb_q(None, None, None, 0, 128, None) == _lib.MLA_OK
    assert lib.mla_up_proj(None, None, None, 0, 128, None) == _lib.MLA_OK


def test_projection_argument_checks(lib):
    assert lib.mla_absorb_q(A, A, A, -1, 128, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(A, A, A, 4, 96, None) == _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_absorb_q(A, None, A, 4, 128, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(A, MIS, A, 4, 128, None) == _lib.MLA_ERR_MISALIGNED
    assert lib.mla_up_proj(MIS, A, A, 4, 128, None) == _lib.MLA_ERR_MISALIGNED
    assert lib.mla_up_proj(A, A, None, 4, 128, None) == _lib.MLA_ERR_INVALID_ARG


def test_fused_and_gather_argument_checks(lib):
    p = _params()
    st = lib.mla_decode(A, A, A, A, A, A, A, A, None, ctypes.byref(p), A, 16, None)
    assert st == _lib.MLA_ERR_WORKSPACE
    st = lib.mla_decode(A, A, MIS, A, A, A, A, A, None, ctypes.byref(p), A, 1 << 30, None)
    assert st == _lib.MLA_ERR_MISALIGNED
    assert lib.mla_gather_kv(A, A, A, None, ctypes.byref(p), None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_gather_kv(MIS, A, A, A2, ctypes.byref(p), None) == _lib.MLA_ERR_MISALIGNED


def test_noalloc_decode_rejects_sizes_beyond_its_array(lib):
    """The allocation-free decode's workspace is a 68 MiB array in the library: more than
    256 workgroups, or too many (sequence, query) units, is refused before any HIP call."""
    def call(p):
        return lib.mla_decode_paged_noalloc(A, A, A, A, A, A, None, ctypes.byref(p), None)
    assert call(_params(num_splits=300)) == _lib.MLA_ERR_UNSUPPORTED
    assert "256 workgroups" in lib.mla_last_error().decode()
    assert call(_params(batch=1 << 16, s_q=256, max_blocks_per_seq=2, num_splits=256)) == _lib.MLA_ERR_UNSUPPORTED
    assert call(_params(page_size=16)) == _lib.MLA_ERR_UNSUPPORTED
    assert call(_params(batch=-1)) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_paged_noalloc(A, A, A, A, A, A, None, None, None) == _lib.MLA_ERR_INVALID_ARG
    assert call(_params(batch=0)) == _lib.MLA_OK


def test_stream_and_workgroup_count_argument_checks(lib):
    p = _params()
    assert lib.mla_decode_num_workgroups(ctypes.byref(p)) == p.num_splits
    assert lib.mla_decode_num_workgroups(ctypes.byref(_params(page_size=16))) == 0
    assert lib.mla_decode_num_workgroups(None) == 0
    need = lib.mla_decode_workspace_size(ctypes.byref(p), 0)
    assert lib.mla_stream_pages(A, A, A, A, ctypes.byref(p), A, need - 1, None) == _lib.MLA_ERR_WORKSPACE
    assert lib.mla_stream_pages(A, A, A, None, ctypes.byref(p), A, need, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_stream_pages(MIS, A, A, A, ctypes.byref(p), A, need, None) == _lib.MLA_ERR_MISALIGNED
    assert lib.mla_stream_pages(A, A, A, ctypes.c_void_p(0x10002), ctypes.byref(p), A, need, None) == \
        _lib.MLA_ERR_MISALIGNED
    assert lib.mla_stream_pages(A, A, A, A, ctypes.byref(_params(num_heads=64)), A, need, None) == \
        _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_stream_pages(None, None, None, None, ctypes.byref(_params(batch=0)), None, 0, None) == _lib.MLA_OK


# ------------------------------------------------------------------ cache append


def _aparams(**kw):
    p = _lib.AppendParams()
    p.batch, p.s_q, p.d_model, p.page_size, p.max_blocks_per_seq = 4, 1, 7168, 64, 8
    p.max_pos, p.num_pages, p.num_heads, p.reserved = 4096, 32, 128, 0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _append(lib, p, ptrs=None, ws=A, ws_bytes=1 << 30, q_r=None):
    x, w, tab, bt, sl, kv = ptrs or (A, A, A, A, A, A)
    return lib.mla_append_kv(x, w, tab, bt, sl, kv, q_r, ctypes.byref(p), ws, ws_bytes, None)


def test_append_params_struct_layout():
    assert ctypes.sizeof(_lib.AppendParams) == 40 and _lib.AppendParams.num_pages.offset == 24
    assert _lib.AppendParams.num_heads.offset == 32


@pytest.mark.parametrize("field,value,status", [
    ("d_model", 7000, _lib.MLA_ERR_UNSUPPORTED), ("d_model", 0, _lib.MLA_ERR_UNSUPPORTED),
    ("d_model", 1 << 17, _lib.MLA_ERR_UNSUPPORTED), ("page_size", 32, _lib.MLA_ERR_UNSUPPORTED),
    ("batch", -1, _lib.MLA_ERR_INVALID_ARG), ("s_q", 0, _lib.MLA_ERR_INVALID_ARG),
    ("max_blocks_per_seq", 0, _lib.MLA_ERR_INVALID_ARG), ("max_pos", 0, _lib.MLA_ERR_INVALID_ARG),
    ("num_pages", 0, _lib.MLA_ERR_INVALID_ARG), ("reserved", 3, _lib.MLA_ERR_INVALID_ARG),
    ("num_heads", 0, _lib.MLA_ERR_INVALID_ARG), ("num_heads", 5000, _lib.MLA_ERR_INVALID_ARG),
])
def test_append_bad_params_rejected(lib, field, value, status):
    p = _aparams(**{field: value})
    assert _append(lib, p) == status
    assert lib.mla_append_workspace_size(ctypes.byref(p)) == 0


def test_append_workspace_size(lib):
    def size(**kw):
        return lib.mla_append_workspace_size(ctypes.byref(_aparams(**kw)))
    C = 0                                             # fp32 partials only
    # decode-sized: 18 column blocks of 32 x 14 splits of the 7168 hidden rows, partials [14, T, 576]
    assert size(batch=64) == C + 14 * 64 * 576 * 4
    assert size(batch=4, s_q=2) == C + 14 * 8 * 576 * 4
    # d = 16384: 32 slabs of 512 rows, 16 splits already give 18 x 16 >= 256 workgroups
    assert size(d_model=16384) == C + 16 * 4 * 576 * 4
    # d = 768 is not a multiple of 512: 64-column blocks, 3 slabs of 256 rows, 3 splits
    assert size(d_model=768) == C + 3 * 4 * 576 * 4
    # 1024 tokens: 16 groups x 9 = 144 workgroups, two splits (a divisor of 28) reach 256
    assert size(batch=1, s_q=1024) == C + 2 * 1024 * 576 * 4
    # prefill-sized: 64 token groups x 9 column blocks fill the chip, one split; the bf16
    # cache then needs no partials, the MXFP8 cache one set (its quantiser runs in the
    # partial-sum kernel), and the size covers both
    assert size(batch=1, s_q=4096) == 1 * 4096 * 576 * 4
    assert size(batch=0) == 16
    assert lib.mla_append_workspace_size(None) == 0


def test_append_argument_checks(lib):
    p = _aparams()
    need = lib.mla_append_workspace_size(ctypes.byref(p))
    assert _append(lib, p, ws_bytes=need - 1) == _lib.MLA_ERR_WORKSPACE
    assert _append(lib, p, ws=None, ws_bytes=need) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_append_kv(A, A, A, A, A, A, None, None, A, need, None) == _lib.MLA_ERR_INVALID_ARG
    for which in range(6):
        ptrs = [A] * 6
        ptrs[which] = None
        assert _append(lib, p, tuple(ptrs)) == _lib.MLA_ERR_INVALID_ARG
        ptrs[which] = MIS if which not in (3, 4) else ctypes.c_void_p(0x10002)
        assert _append(lib, p, tuple(ptrs)) == _lib.MLA_ERR_MISALIGNED
    assert _append(lib, p, ws=MIS) == _lib.MLA_ERR_MISALIGNED
    assert _append(lib, p, q_r=MIS) == _lib.MLA_ERR_MISALIGNED
    assert _append(lib, _aparams(batch=0), (None,) * 6, ws=None, ws_bytes=0) == _lib.MLA_OK


def test_mxfp8_argument_checks(lib):
    q = lib.mla_quantize_kv_mxfp8
    assert q(A, A, -1, None) == _lib.MLA_ERR_INVALID_ARG
    assert q(None, None, 0, None) == _lib.MLA_OK
    assert q(None, A, 4, None) == _lib.MLA_ERR_INVALID_ARG
    assert q(A, MIS, 4, None) == _lib.MLA_ERR_MISALIGNED
    p = _params()
    dp = lib.mla_decode_paged_mxfp8
    assert dp(A, A, A, A, A, A, None, ctypes.byref(_params(s_q=257)), A, 1 << 30, None) == _lib.MLA_ERR_UNSUPPORTED
    assert dp(A, A, None, A, A, A, None, ctypes.byref(p), A, 1 << 30, None) == _lib.MLA_ERR_INVALID_ARG
    assert dp(A, A, MIS, A, A, A, None, ctypes.byref(p), A, 1 << 30, None) == _lib.MLA_ERR_MISALIGNED
    assert dp(A, A, A, A, A, A, None, ctypes.byref(p), A, 16, None) == _lib.MLA_ERR_WORKSPACE
    assert dp(None, None, None, None, None, None, None, ctypes.byref(_params(batch=0)), None, 0, None) == _lib.MLA_OK
    fd = lib.mla_decode_mxfp8
    assert fd(A, A, A, A, None, A, A, A, None, ctypes.byref(p), A, 1 << 30, None) == _lib.MLA_ERR_INVALID_ARG
    assert fd(A, A, A, A, MIS, A, A, A, None, ctypes.byref(p), A, 1 << 30, None) == _lib.MLA_ERR_MISALIGNED
    assert fd(A, A, A, A, A, A, A, A, None, ctypes.byref(p), A, 16, None) == _lib.MLA_ERR_WORKSPACE
    ap = _aparams()
    aq = lib.mla_append_kv_mxfp8
    assert aq(A, A, A, A, A, None, None, ctypes.byref(ap), A, 1 << 30, None) == _lib.MLA_ERR_INVALID_ARG
    assert aq(A, A, A, A, A, MIS, None, ctypes.byref(ap), A, 1 << 30, None) == _lib.MLA_ERR_MISALIGNED
    assert aq(A, A, A, A, A, A, None, ctypes.byref(_aparams(d_model=100)), A, 1 << 30, None) == \
        _lib.MLA_ERR_UNSUPPORTED


def test_rope_argument_checks(lib):
    assert lib.mla_rope_q(A, A, A, -1, 1, 128, 10, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_q(A, A, A, 1, 0, 128, 10, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_q(A, A, A, 1, 1, 0, 10, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_q(A, A, A, 1, 1, 128, 0, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_q(A, None, A, 1, 1, 128, 10, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_q(MIS, A, A, 1, 1, 128, 10, None) == _lib.MLA_ERR_MISALIGNED
    assert lib.mla_rope_q(A, A, ctypes.c_void_p(0x10002), 1, 1, 128, 10, None) == _lib.MLA_ERR_MISALIGNED
    assert lib.mla_rope_q(None, None, None, 0, 1, 128, 10, None) == _lib.MLA_OK
    assert lib.mla_rope_table(A, 0, 10000.0, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_table(A, 10, 1.0, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_table(A, 10, float("nan"), None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_table(None, 10, 10000.0, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_table(MIS, 10, 10000.0, None) == _lib.MLA_ERR_MISALIGNED


# ------------------------------------------------------------------ prefill


def _pparams(**kw):
    p = _lib.PrefillParams()
    p.batch, p.s_q, p.num_heads, p.page_size, p.max_blocks_per_seq = 2, 512, 128, 64, 16
    p.mode, p.num_pages, p.scale, p.threshold, p.reserved = 0, 64, 0.0721687836, 0, 0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _prefill(lib, p, ws=A, ws_bytes=1 << 40, ptrs=None):
    q, r, wk, wv, kv, bt, sl, out, lse = ptrs or (A, A, A, A, A, A, A, A, None)
    return lib.mla_prefill(q, r, wk, wv, kv, bt, sl, out, lse, ctypes.byref(p), ws, ws_bytes, None)


def test_prefill_params_struct_layout():
    assert ctypes.sizeof(_lib.PrefillParams) == 48 and _lib.PrefillParams.num_pages.offset == 24
    assert _lib.PrefillParams.threshold.offset == 36 and _lib.PrefillParams.reserved.offset == 40


@pytest.mark.parametrize("field,value,status", [
    ("num_heads", 64, _lib.MLA_ERR_UNSUPPORTED), ("page_size", 32, _lib.MLA_ERR_UNSUPPORTED),
    ("batch", -1, _lib.MLA_ERR_INVALID_ARG), ("s_q", 0, _lib.MLA_ERR_INVALID_ARG),
    ("mode", 3, _lib.MLA_ERR_INVALID_ARG), ("threshold", 300, _lib.MLA_ERR_INVALID_ARG),
    ("scale", 0.0, _lib.MLA_ERR_INVALID_ARG), ("num_pages", 0, _lib.MLA_ERR_INVALID_ARG),
    ("max_blocks_per_seq", 0, _lib.MLA_ERR_INVALID_ARG), ("reserved", 1, _lib.MLA_ERR_INVALID_ARG),
])
def test_prefill_bad_params_rejected(lib, field, value, status):
    p = _pparams(**{field: value})
    assert _prefill(lib, p) == status
    assert lib.mla_prefill_workspace_size(ctypes.byref(p)) == 0


def test_prefill_branch_and_workspace(lib):
    # s_q >= 256: decompress, K and V of 2 x 16 x 64 token slots x 128 heads x 128 bf16 each
    expanded = 2 * 16 * 64 * 128 * 128 * 2
    assert lib.mla_prefill_workspace_size(ctypes.byref(_pparams())) == 2 * expanded
    # s_q < 256: the absorbed decode's workspace
    d = _params(batch=2, s_q=100, max_blocks_per_seq=16, num_pages=64, num_splits=0)
    assert lib.mla_prefill_workspace_size(ctypes.byref(_pparams(s_q=100))) == lib.mla_decode_workspace_size(
        ctypes.byref(d), 1)
    # forced absorption of a chunk longer than 256 is unsupported; forced decompression of a short one is fine
    assert _prefill(lib, _pparams(mode=1)) == _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_prefill_workspace_size(ctypes.byref(_pparams(s_q=10, mode=2))) == 2 * expanded
    # a lower threshold moves short chunks to decompression
    assert lib.mla_prefill_workspace_size(ctypes.byref(_pparams(s_q=100, threshold=64))) == 2 * expanded
    assert _prefill(lib, _pparams(), ws_bytes=2 * expanded - 1) == _lib.MLA_ERR_WORKSPACE
    assert _prefill(lib, _pparams(), ptrs=(A, A, MIS, A, A, A, A, A, None)) == _lib.MLA_ERR_MISALIGNED
    assert _prefill(lib, _pparams(), ptrs=(A, None, A, A, A, A, A, A, None)) == _lib.MLA_ERR_INVALID_ARG
    assert _prefill(lib, _pparams(batch=0), ws=None, ws_bytes=0, ptrs=(None,) * 8 + (None,)) == _lib.MLA_OK

"""Absorbed MLA decode over a paged latent cache on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libmla_kv04.so`` (see include/mla.h).
Tensors are torch tensors on the current HIP device: bf16 (or int16/uint16 bit
views) for activations, weights and the cache, int32 for block tables and
lengths.  Every call enqueues HIP kernels on the current torch stream; torch is
used only for device memory and streams.
"""

from __future__ import annotations

import ctypes
import math

from . import _lib
from ._lib import AppendParams, DecodeParams, MlaError, PrefillParams  # noqa: F401

NUM_HEADS = 128
D_HC = 128
D_C = 512
D_R = 64
PAGE = 64
DEFAULT_SCALE = 1.0 / math.sqrt(D_HC + D_R)

__all__ = [
    "absorb_q", "decode_paged", "up_proj", "decode", "gather_kv", "workspace_size", "make_params",
    "device_cu_count", "MlaError", "DecodeParams", "KernelTimer", "AppendParams", "append_kv",
    "append_workspace", "append_workspace_size", "make_append_params", "rope_q", "rope_table",
    "PrefillParams", "make_prefill_params", "prefill", "prefill_workspace_size", "PREFILL_THRESHOLD",
    "MXFP8_ROW_BYTES", "quantize_kv_mxfp8", "decode_paged_mxfp8", "decode_mxfp8", "append_kv_mxfp8",
    "decode_num_workgroups", "stream_pages",
]

MXFP8_ROW_BYTES = 656    # MXFP8 cache row: 512 E4M3 codes, 16 E8M0 scale bytes, 64 bf16 of k_R

PREFILL_THRESHOLD = 256


def _torch():
    import torch
    return torch


def _stream() -> int:
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _ptr(t, name, dtypes, shape=None):
    torch = _torch()
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _i32():
    return (_torch().int32,)


def make_params(batch: int, s_q: int, max_blocks_per_seq: int, num_pages: int, scale: float = DEFAULT_SCALE,
                num_splits: int = 0) -> DecodeParams:
    p = DecodeParams()
    p.batch, p.s_q, p.num_heads, p.page_size = batch, s_q, NUM_HEADS, PAGE
    p.max_blocks_per_seq, p.num_splits, p.num_pages, p.scale, p.reserved = (
        max_blocks_per_seq, num_splits, num_pages, scale, 0)
    return p


def device_cu_count() -> int:
    lib = _lib.load()
    n = ctypes.c_int32(0)
    _lib.check(lib.mla_device_cu_count(ctypes.byref(n)), "mla_device_cu_count")
    return int(n.value)


def workspace_size(params: DecodeParams, fused: bool = False) -> int:
    lib = _lib.load()
    n = lib.mla_decode_workspace_size(ctypes.byref(params), 1 if fused else 0)
    if n == 0:
        raise MlaError(_lib.MLA_ERR_INVALID_ARG, "mla_decode_workspace_size", lib.mla_last_error().decode())
    return int(n)


def _workspace(params, fused, workspace):
    torch = _torch()
    need = workspace_size(params, fused)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
    return workspace, need


def absorb_q(q_c, w_uk, out=None):
    """q_abs[t, h, :] = q_c[t, h, :] . W_UK[h];  q_c [..., 128, 128], w_uk [128, 128, 512]."""
    torch = _torch()
    lead = q_c.shape[:-2]
    tokens = int(math.prod(lead))
    if out is None:
        out = torch.empty(*lead, NUM_HEADS, D_C, dtype=torch.bfloat16, device=q_c.device)
    lib = _lib.load()
    st = lib.mla_absorb_q(_ptr(q_c, "q_c", _bf16_types(), (*lead, NUM_HEADS, D_HC)),
                          _ptr(w_uk, "w_uk", _bf16_types(), (NUM_HEADS, D_HC, D_C)),
                          _ptr(out, "q_abs", _bf16_types(), (*lead, NUM_HEADS, D_C)), tokens, NUM_HEADS, _stream())
    _lib.check(st, "mla_absorb_q")
    return out


def up_proj(out_latent, w_uv, out=None):
    """out[t, h, :] = out_latent[t, h, :] . W_UV[h];  w_uv [128, 512, 128]."""
    torch = _torch()
    lead = out_latent.shape[:-2]
    tokens = int(math.prod(lead))
    if out is None:
        out = torch.empty(*lead, NUM_HEADS, D_HC, dtype=torch.bfloat16, device=out_latent.device)
    lib = _lib.load()
    st = lib.mla_up_proj(_ptr(out_latent, "out_latent", _bf16_types(), (*lead, NUM_HEADS, D_C)),
                         _ptr(w_uv, "w_uv", _bf16_types(), (NUM_HEADS, D_C, D_HC)),
                         _ptr(out, "out", _bf16_types(), (*lead, NUM_HEADS, D_HC)), tokens, NUM_HEADS, _stream())
    _lib.check(st, "mla_up_proj")
    return out


def _kv_arg(kv, P, mxfp8):
    torch = _torch()
    if mxfp8:
        return _ptr(kv, "kv_mxfp8", (torch.uint8,), (P, PAGE, MXFP8_ROW_BYTES))
    return _ptr(kv, "kv_blocks", _bf16_types(), (P, PAGE, D_C + D_R))


def _decode_paged(q_abs, q_r, kv, block_table, seqlens, scale, num_splits, out_latent, lse, want_lse, workspace,
                  mxfp8):
    torch = _torch()
    B, s_q = int(q_abs.shape[0]), int(q_abs.shape[1])
    P = int(kv.shape[0])
    mb = int(block_table.shape[1])
    params = make_params(B, s_q, mb, P, scale, num_splits)
    if out_latent is None:
        out_latent = torch.empty(B, s_q, NUM_HEADS, D_C, dtype=torch.bfloat16, device=q_abs.device)
    if lse is None and want_lse:
        lse = torch.empty(B, s_q, NUM_HEADS, dtype=torch.float32, device=q_abs.device)
    workspace, need = _workspace(params, False, workspace)
    lib = _lib.load()
    fn, name = (lib.mla_decode_paged_mxfp8, "mla_decode_paged_mxfp8") if mxfp8 else \
        (lib.mla_decode_paged, "mla_decode_paged")
    st = fn(
        _ptr(q_abs, "q_abs", _bf16_types(), (B, s_q, NUM_HEADS, D_C)),
        _ptr(q_r, "q_r", _bf16_types(), (B, s_q, NUM_HEADS, D_R)),
        _kv_arg(kv, P, mxfp8),
        _ptr(block_table, "block_table", _i32(), (B, mb)), _ptr(seqlens, "seqlens", _i32(), (B,)),
        _ptr(out_latent, "out_latent", _bf16_types(), (B, s_q, NUM_HEADS, D_C)),
        _ptr(lse, "lse", (torch.float32,), (B, s_q, NUM_HEADS)), ctypes.byref(params),
        _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream())
    _lib.check(st, name)
    return out_latent, lse


def decode_paged(q_abs, q_r, kv_blocks, block_table, seqlens, *, scale=DEFAULT_SCALE, num_splits=0,
                 out_latent=None, lse=None, want_lse=True, workspace=None):
    """Paged latent-space decode.  q_abs [B, s_q, 128, 512], q_r [B, s_q, 128, 64],
    kv_blocks [P, 64, 576], block_table [B, max_blocks] int32, seqlens [B] int32.
    Returns (out_latent [B, s_q, 128, 512] bf16, lse [B, s_q, 128] fp32 or None)."""
    return _decode_paged(q_abs, q_r, kv_blocks, block_table, seqlens, scale, num_splits, out_latent, lse, want_lse,
                         workspace, False)


def decode_paged_mxfp8(q_abs, q_r, kv_mxfp8, block_table, seqlens, *, scale=DEFAULT_SCALE, num_splits=0,
                       out_latent=None, lse=None, want_lse=True, workspace=None):
    """decode_paged over an MXFP8 cache: kv_mxfp8 [P, 64, 656] uint8 (rows of mla.h)."""
    return _decode_paged(q_abs, q_r, kv_mxfp8, block_table, seqlens, scale, num_splits, out_latent, lse, want_lse,
                         workspace, True)


def _decode(q_c, q_r, w_uk, w_uv, kv, block_table, seqlens, scale, num_splits, out, lse, want_lse, workspace,
            mxfp8):
    torch = _torch()
    B, s_q = int(q_c.shape[0]), int(q_c.shape[1])
    P = int(kv.shape[0])
    mb = int(block_table.shape[1])
    params = make_params(B, s_q, mb, P, scale, num_splits)
    if out is None:
        out = torch.empty(B, s_q, NUM_HEADS, D_HC, dtype=torch.bfloat16, device=q_c.device)
    if lse is None and want_lse:
        lse = torch.empty(B, s_q, NUM_HEADS, dtype=torch.float32, device=q_c.device)
    workspace, need = _workspace(params, True, workspace)
    lib = _lib.load()
    fn, name = (lib.mla_decode_mxfp8, "mla_decode_mxfp8") if mxfp8 else (lib.mla_decode, "mla_decode")
    st = fn(
        _ptr(q_c, "q_c", _bf16_types(), (B, s_q, NUM_HEADS, D_HC)),
        _ptr(q_r, "q_r", _bf16_types(), (B, s_q, NUM_HEADS, D_R)),
        _ptr(w_uk, "w_uk", _bf16_types(), (NUM_HEADS, D_HC, D_C)),
        _ptr(w_uv, "w_uv", _bf16_types(), (NUM_HEADS, D_C, D_HC)),
        _kv_arg(kv, P, mxfp8),
        _ptr(block_table, "block_table", _i32(), (B, mb)), _ptr(seqlens, "seqlens", _i32(), (B,)),
        _ptr(out, "out", _bf16_types(), (B, s_q, NUM_HEADS, D_HC)),
        _ptr(lse, "lse", (torch.float32,), (B, s_q, NUM_HEADS)), ctypes.byref(params),
        _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream())
    _lib.check(st, name)
    return out, lse


def decode(q_c, q_r, w_uk, w_uv, kv_blocks, block_table, seqlens, *, scale=DEFAULT_SCALE, num_splits=0, out=None,
           lse=None, want_lse=True, workspace=None):
    """Fused decode step (absorb -> paged decode -> merge -> up-projection).
    Returns (out [B, s_q, 128, 128] bf16, lse [B, s_q, 128] fp32 or None)."""
    return _decode(q_c, q_r, w_uk, w_uv, kv_blocks, block_table, seqlens, scale, num_splits, out, lse, want_lse,
                   workspace, False)


def decode_mxfp8(q_c, q_r, w_uk, w_uv, kv_mxfp8, block_table, seqlens, *, scale=DEFAULT_SCALE, num_splits=0,
                 out=None, lse=None, want_lse=True, workspace=None):
    """The fused decode step over an MXFP8 cache (kv_mxfp8 [P, 64, 656] uint8)."""
    return _decode(q_c, q_r, w_uk, w_uv, kv_mxfp8, block_table, seqlens, scale, num_splits, out, lse, want_lse,
                   workspace, True)


def quantize_kv_mxfp8(kv_blocks, out=None):
    """MXFP8 cache [P, 64, 656] uint8 from a bf16 cache [P, 64, 576] (every row)."""
    torch = _torch()
    P = int(kv_blocks.shape[0])
    if out is None:
        out = torch.empty(P, PAGE, MXFP8_ROW_BYTES, dtype=torch.uint8, device=kv_blocks.device)
    lib = _lib.load()
    st = lib.mla_quantize_kv_mxfp8(_ptr(kv_blocks, "kv_blocks", _bf16_types(), (P, PAGE, D_C + D_R)),
                                   _ptr(out, "kv_mxfp8", (torch.uint8,), (P, PAGE, MXFP8_ROW_BYTES)), P, _stream())
    _lib.check(st, "mla_quantize_kv_mxfp8")
    return out


class KernelTimer:
    """Per-kernel HIP-event timing of decode and cache-append calls (library hook; see
    mla_profile_enable).

    with KernelTimer() as kt: ...calls...;  kt.ms -> dict of summed milliseconds per kernel of
    decode calls, holding only kernels that were launched, kt.launches -> how many calls
    launched each of them, kt.calls; kt.per_launch_ms() -> average milliseconds per launch;
    kt.append_ms, kt.append_calls likewise for append calls."""

    NAMES = ("absorb", "plan", "decode", "combine", "up_proj")

    def __enter__(self):
        lib = _lib.load()
        _lib.check(lib.mla_profile_enable(1), "mla_profile_enable")
        return self

    APPEND_NAMES = ("append_proj", "append_sum")
    PREFILL_NAMES = ("decompress", "attention")

    def __exit__(self, *exc):
        lib = _lib.load()
        ms = (ctypes.c_double * 5)()
        launches = (ctypes.c_int32 * 5)()
        calls = ctypes.c_int32(0)
        st = lib.mla_profile_collect(ms, launches, ctypes.byref(calls))
        ams = (ctypes.c_double * 2)()
        acalls = ctypes.c_int32(0)
        st2 = lib.mla_profile_collect_append(ams, ctypes.byref(acalls))
        pms = (ctypes.c_double * 2)()
        pcalls = ctypes.c_int32(0)
        st3 = lib.mla_profile_collect_prefill(pms, ctypes.byref(pcalls))
        lib.mla_profile_enable(0)
        _lib.check(st3, "mla_profile_collect_prefill")
        self.prefill_ms = dict(zip(self.PREFILL_NAMES, list(pms)))
        self.prefill_calls = int(pcalls.value)
        _lib.check(st, "mla_profile_collect")
        _lib.check(st2, "mla_profile_collect_append")
        self.launches = {k: int(n) for k, n in zip(self.NAMES, list(launches)) if n > 0}
        self.ms = {k: v for k, v in zip(self.NAMES, list(ms)) if k in self.launches}
        self.calls = int(calls.value)
        self.append_ms = dict(zip(self.APPEND_NAMES, list(ams)))
        self.append_calls = int(acalls.value)
        return False

    def per_launch_ms(self):
        """Average milliseconds per launch of each decode-call kernel that ran."""
        return {k: v / self.launches[k] for k, v in self.ms.items()}


def decode_num_workgroups(params: DecodeParams) -> int:
    """Split-KV workgroups a decode with these parameters launches."""
    lib = _lib.load()
    n = lib.mla_decode_num_workgroups(ctypes.byref(params))
    if n <= 0:
        raise MlaError(_lib.MLA_ERR_INVALID_ARG, "mla_decode_num_workgroups", lib.mla_last_error().decode())
    return int(n)


def stream_pages(kv_blocks, block_table, seqlens, *, s_q=1, num_splits=0, sums=None, workspace=None):
    """The decode's page stream alone (mla_stream_pages): reads every cache row a decode
    over these sequences reads, with the decode's split, loads and LDS ring, and no
    arithmetic.  Returns sums [workgroups * 256] uint32 (see include/mla.h)."""
    torch = _torch()
    B = int(block_table.shape[0])
    mb = int(block_table.shape[1])
    P = int(kv_blocks.shape[0])
    params = make_params(B, s_q, mb, P, DEFAULT_SCALE, num_splits)
    n = decode_num_workgroups(params) * 256
    if sums is None:
        sums = torch.empty(n, dtype=torch.int32, device=kv_blocks.device)
    workspace, need = _workspace(params, False, workspace)
    lib = _lib.load()
    st = lib.mla_stream_pages(_ptr(kv_blocks, "kv_blocks", _bf16_types(), (P, PAGE, D_C + D_R)),
                              _ptr(block_table, "block_table", _i32(), (B, mb)),
                              _ptr(seqlens, "seqlens", _i32(), (B,)),
                              _ptr(sums, "sums", (torch.int32,), (n,)), ctypes.byref(params),
                              _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream())
    _lib.check(st, "mla_stream_pages")
    return sums


def gather_kv(kv_blocks, block_table, seqlens, out=None):
    """Dense copy of the paged cache: [B, max_blocks * 64, 576], zero past each length."""
    torch = _torch()
    B = int(block_table.shape[0])
    mb = int(block_table.shape[1])
    P = int(kv_blocks.shape[0])
    if out is None:
        out = torch.empty(B, mb * PAGE, D_C + D_R, dtype=torch.bfloat16, device=kv_blocks.device)
    params = make_params(B, 1, mb, P)
    lib = _lib.load()
    st = lib.mla_gather_kv(_ptr(kv_blocks, "kv_blocks", _bf16_types(), (P, PAGE, D_C + D_R)),
                           _ptr(block_table, "block_table", _i32(), (B, mb)), _ptr(seqlens, "seqlens", _i32(), (B,)),
                           _ptr(out, "dense", _bf16_types(), (B, mb * PAGE, D_C + D_R)), ctypes.byref(params),
                           _stream())
    _lib.check(st, "mla_gather_kv")
    return out


# ------------------------------------------------------------------ cache append


def make_append_params(batch: int, s_q: int, d_model: int, max_blocks_per_seq: int, num_pages: int,
                       max_pos: int, num_heads: int = NUM_HEADS) -> AppendParams:
    p = AppendParams()
    p.batch, p.s_q, p.d_model, p.page_size = batch, s_q, d_model, PAGE
    p.max_blocks_per_seq, p.max_pos, p.num_pages = max_blocks_per_seq, max_pos, num_pages
    p.num_heads, p.reserved = num_heads, 0
    return p


def append_workspace_size(params: AppendParams) -> int:
    lib = _lib.load()
    n = lib.mla_append_workspace_size(ctypes.byref(params))
    if n == 0:
        raise MlaError(_lib.MLA_ERR_INVALID_ARG, "mla_append_workspace_size", lib.mla_last_error().decode())
    return int(n)


def rope_table(max_pos: int, base: float = 10000.0, out=None):
    """fp32 rotary table [max_pos, 64]: cosines then sines of p * base^(-2i/64)."""
    torch = _torch()
    if out is None:
        out = torch.empty(max_pos, D_R, dtype=torch.float32, device="cuda")
    lib = _lib.load()
    st = lib.mla_rope_table(_ptr(out, "rope_table", (torch.float32,), (max_pos, D_R)), max_pos, float(base), _stream())
    _lib.check(st, "mla_rope_table")
    return out


def append_workspace(params: AppendParams):
    """A workspace for mla_append_kv (no initialisation needed)."""
    return _torch().empty(append_workspace_size(params), dtype=_torch().uint8, device="cuda")


def _append(x, w_a, table, kv, block_table, seqlens, q_r, workspace, mxfp8):
    torch = _torch()
    B, s_q, d = (int(v) for v in x.shape)
    P = int(kv.shape[0])
    mb = int(block_table.shape[1])
    max_pos = int(table.shape[0])
    H = int(q_r.shape[2]) if q_r is not None else NUM_HEADS
    params = make_append_params(B, s_q, d, mb, P, max_pos, H)
    if workspace is None:
        workspace = append_workspace(params)
    lib = _lib.load()
    fn, name = (lib.mla_append_kv_mxfp8, "mla_append_kv_mxfp8") if mxfp8 else (lib.mla_append_kv, "mla_append_kv")
    st = fn(
        _ptr(x, "x", _bf16_types(), (B, s_q, d)), _ptr(w_a, "w_a", _bf16_types(), (d, D_C + D_R)),
        _ptr(table, "table", (torch.float32,), (max_pos, D_R)),
        _ptr(block_table, "block_table", _i32(), (B, mb)), _ptr(seqlens, "seqlens", _i32(), (B,)),
        _kv_arg(kv, P, mxfp8),
        _ptr(q_r, "q_r", _bf16_types(), (B, s_q, H, D_R)), ctypes.byref(params),
        _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream())
    _lib.check(st, name)
    return kv


def append_kv(x, w_a, table, kv_blocks, block_table, seqlens, *, q_r=None, workspace=None):
    """Writes the rows of the new tokens into the paged cache (in place).

    x [B, s_q, d] bf16, w_a [d, 576] bf16 (W_DKV | W_KR), table [max_pos, 64] fp32,
    kv_blocks [P, 64, 576], block_table [B, max_blocks] int32, seqlens [B] int32
    (including the new tokens).  q_r [B, s_q, H, 64] bf16, when given, is rotated in
    place by the same call.  A workspace passed in is reused only on one stream.
    Returns kv_blocks."""
    return _append(x, w_a, table, kv_blocks, block_table, seqlens, q_r, workspace, False)


def append_kv_mxfp8(x, w_a, table, kv_mxfp8, block_table, seqlens, *, q_r=None, workspace=None):
    """append_kv into an MXFP8 cache (kv_mxfp8 [P, 64, 656] uint8, in place)."""
    return _append(x, w_a, table, kv_mxfp8, block_table, seqlens, q_r, workspace, True)


def rope_q(q_r, table, seqlens):
    """Rotates q_r [B, s_q, H, 64] (bf16) in place to positions seqlens[b] - s_q + i."""
    torch = _torch()
    B, s_q, H = int(q_r.shape[0]), int(q_r.shape[1]), int(q_r.shape[2])
    max_pos = int(table.shape[0])
    lib = _lib.load()
    st = lib.mla_rope_q(_ptr(q_r, "q_r", _bf16_types(), (B, s_q, H, D_R)),
                        _ptr(table, "table", (torch.float32,), (max_pos, D_R)),
                        _ptr(seqlens, "seqlens", _i32(), (B,)), B, s_q, H, max_pos, _stream())
    _lib.check(st, "mla_rope_q")
    return q_r


# ------------------------------------------------------------------ prefill


def make_prefill_params(batch: int, s_q: int, max_blocks_per_seq: int, num_pages: int, scale: float = DEFAULT_SCALE,
                        mode: int = 0, threshold: int = 0) -> PrefillParams:
    p = PrefillParams()
    p.batch, p.s_q, p.num_heads, p.page_size = batch, s_q, NUM_HEADS, PAGE
    p.max_blocks_per_seq, p.mode, p.num_pages, p.scale = max_blocks_per_seq, mode, num_pages, scale
    p.threshold, p.reserved = threshold, 0
    return p


def prefill_workspace_size(params: PrefillParams) -> int:
    lib = _lib.load()
    n = lib.mla_prefill_workspace_size(ctypes.byref(params))
    if n == 0:
        raise MlaError(_lib.MLA_ERR_INVALID_ARG, "mla_prefill_workspace_size", lib.mla_last_error().decode())
    return int(n)


def prefill(q_c, q_r, w_uk, w_uv, kv_blocks, block_table, seqlens, *, scale=DEFAULT_SCALE, mode=0, threshold=0,
            out=None, lse=None, want_lse=True, workspace=None):
    """Attention of a chunk of s_q new tokens per sequence (rows already cached).

    q_c [B, s_q, 128, 128], q_r [B, s_q, 128, 64]; mode 0 picks the decompress branch
    for s_q >= threshold (256 by default) and absorption below it, 1 forces
    absorption, 2 forces decompression.  Returns (out [B, s_q, 128, 128] bf16, lse)."""
    torch = _torch()
    B, s_q = int(q_c.shape[0]), int(q_c.shape[1])
    P = int(kv_blocks.shape[0])
    mb = int(block_table.shape[1])
    params = make_prefill_params(B, s_q, mb, P, scale, mode, threshold)
    if out is None:
        out = torch.empty(B, s_q, NUM_HEADS, D_HC, dtype=torch.bfloat16, device=q_c.device)
    if lse is None and want_lse:
        lse = torch.empty(B, s_q, NUM_HEADS, dtype=torch.float32, device=q_c.device)
    if workspace is None:
        workspace = torch.empty(prefill_workspace_size(params), dtype=torch.uint8, device=q_c.device)
    lib = _lib.load()
    st = lib.mla_prefill(
        _ptr(q_c, "q_c", _bf16_types(), (B, s_q, NUM_HEADS, D_HC)),
        _ptr(q_r, "q_r", _bf16_types(), (B, s_q, NUM_HEADS, D_R)),
        _ptr(w_uk, "w_uk", _bf16_types(), (NUM_HEADS, D_HC, D_C)),
        _ptr(w_uv, "w_uv", _bf16_types(), (NUM_HEADS, D_C, D_HC)),
        _ptr(kv_blocks, "kv_blocks", _bf16_types(), (P, PAGE, D_C + D_R)),
        _ptr(block_table, "block_table", _i32(), (B, mb)), _ptr(seqlens, "seqlens", _i32(), (B,)),
        _ptr(out, "out", _bf16_types(), (B, s_q, NUM_HEADS, D_HC)),
        _ptr(lse, "lse", (torch.float32,), (B, s_q, NUM_HEADS)), ctypes.byref(params),
        _ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream())
    _lib.check(st, "mla_prefill")
    return out, lse

"""ctypes view of the C ABI declared in include/mla.h (libmla_kv04.so).

Argument marshalling only: every computation runs in the HIP kernels of the
library.  Loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_kv04.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_MISALIGNED = 2
MLA_ERR_UNSUPPORTED = 3
MLA_ERR_WORKSPACE = 4
MLA_ERR_HIP = 5

# Every symbol include/mla.h declares; tests check they are all exported.
EXPORTS = (
    "mla_absorb_q",
    "mla_decode_workspace_size",
    "mla_decode_paged",
    "mla_up_proj",
    "mla_decode",
    "mla_gather_kv",
    "mla_append_workspace_size",
    "mla_append_kv",
    "mla_rope_q",
    "mla_rope_table",
    "mla_profile_enable",
    "mla_profile_collect",
    "mla_profile_collect_append",
    "mla_profile_collect_prefill",
    "mla_prefill_workspace_size",
    "mla_prefill",
    "mla_device_cu_count",
    "mla_quantize_kv_mxfp8",
    "mla_decode_paged_mxfp8",
    "mla_decode_mxfp8",
    "mla_append_kv_mxfp8",
    "mla_decode_paged_noalloc",
    "mla_decode_num_workgroups",
    "mla_stream_pages",
    "mla_status_string",
    "mla_last_error",
)


class DecodeParams(ctypes.Structure):
    """Mirror of ``mla_decode_params``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("s_q", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


class AppendParams(ctypes.Structure):
    """Mirror of ``mla_append_params``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("s_q", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_pos", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("num_heads", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class PrefillParams(ctypes.Structure):
    """Mirror of ``mla_prefill_params``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("s_q", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("threshold", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the library once; raise if it is missing (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_04_amd.build` "
            "(the MLA decode path has no CPU fallback)")
    # torch first: the library registers its kernels with the HIP runtime when it is
    # opened, and the process must use one runtime -- the one torch brings for the
    # device memory and streams the library works on.  Opened the other way round
    # (library, then torch) the library's calls found no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pp = ctypes.POINTER(DecodeParams)
    ap = ctypes.POINTER(AppendParams)
    fp = ctypes.POINTER(PrefillParams)
    sigs = {
        "mla_absorb_q": ([vp, vp, vp, i32, i32, vp], ctypes.c_int),
        "mla_decode_workspace_size": ([pp, i32], sz),
        "mla_decode_paged": ([vp, vp, vp, vp, vp, vp, vp, pp, vp, sz, vp], ctypes.c_int),
        "mla_up_proj": ([vp, vp, vp, i32, i32, vp], ctypes.c_int),
        "mla_decode": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, pp, vp, sz, vp], ctypes.c_int),
        "mla_gather_kv": ([vp, vp, vp, vp, pp, vp], ctypes.c_int),
        "mla_append_workspace_size": ([ap], sz),
        "mla_append_kv": ([vp, vp, vp, vp, vp, vp, vp, ap, vp, sz, vp], ctypes.c_int),
        "mla_rope_q": ([vp, vp, vp, i32, i32, i32, i32, vp], ctypes.c_int),
        "mla_rope_table": ([vp, i32, ctypes.c_double, vp], ctypes.c_int),
        "mla_device_cu_count": ([ctypes.POINTER(i32)], ctypes.c_int),
        "mla_profile_enable": ([i32], ctypes.c_int),
        "mla_profile_collect": ([ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32), ctypes.POINTER(i32)],
                                ctypes.c_int),
        "mla_profile_collect_append": ([ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)], ctypes.c_int),
        "mla_profile_collect_prefill": ([ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)], ctypes.c_int),
        "mla_prefill_workspace_size": ([fp], sz),
        "mla_prefill": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, fp, vp, sz, vp], ctypes.c_int),
        "mla_quantize_kv_mxfp8": ([vp, vp, ctypes.c_int64, vp], ctypes.c_int),
        "mla_decode_paged_mxfp8": ([vp, vp, vp, vp, vp, vp, vp, pp, vp, sz, vp], ctypes.c_int),
        "mla_decode_mxfp8": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, pp, vp, sz, vp], ctypes.c_int),
        "mla_append_kv_mxfp8": ([vp, vp, vp, vp, vp, vp, vp, ap, vp, sz, vp], ctypes.c_int),
        "mla_decode_paged_noalloc": ([vp, vp, vp, vp, vp, vp, vp, pp, vp], ctypes.c_int),
        "mla_decode_num_workgroups": ([pp], i32),
        "mla_stream_pages": ([vp, vp, vp, vp, pp, vp, sz, vp], ctypes.c_int),
        "mla_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "mla_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != MLA_OK:
        lib = load()
        detail = lib.mla_last_error().decode() or lib.mla_status_string(status).decode()
        raise MlaError(status, where, detail)

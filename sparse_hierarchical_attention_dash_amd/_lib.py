"""ctypes binding of libdash.so (include/dash.h).

Argument marshalling only: every step of the forward path runs in the HIP
library.  If the library has not been built this module raises on first use;
there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdash.so")

DASH_OK = 0
DASH_ERR_INVALID_ARGUMENT = 1
DASH_ERR_UNSUPPORTED = 2
DASH_ERR_WORKSPACE_TOO_SMALL = 3
DASH_ERR_HIP = 4

DASH_F32 = 0
DASH_BF16 = 1

DASH_OP_SUMMARIZE = 0
DASH_OP_ROUTE = 1
DASH_OP_PREFILL = 2
DASH_OP_DECODE = 3
DASH_OP_SPARSE = 4
DASH_OP_DECODE_SPARSE = 5
DASH_OP_ROUTE_DECODE = 6
DASH_OP_BACKWARD = 7
DASH_OP_PREFILL_BACKWARD = 8
DASH_NOALLOC_SCRATCH_BYTES = 32 << 20   # include/dash.h

EXPORTED = ("dash_get_layout", "dash_summarize", "dash_route", "dash_attn_prefill",
            "dash_attn_sparse", "dash_attn_decode", "dash_route_topk", "dash_attn_decode_sparse",
            "dash_cache_append", "dash_summarize_diagonal", "dash_attn_sparse_backward",
            "dash_attn_prefill_backward", "dash_attn_decode_noalloc", "dash_noalloc_scratch_need", "dash_probe_peak",
            "dash_prefill_schedule", "dash_attn_decode_append",
            "dash_workspace_size", "dash_status_string", "dash_abi_version")


class DashShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("cu_seqlens", ctypes.c_void_p),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class DashLayout(ctypes.Structure):
    _fields_ = [
        ("summary_rows", ctypes.c_int64),
        ("chunk_slots", ctypes.c_int32),
        ("mask_words", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
    ]


class DashError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_F = ctypes.c_float
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SHAPE = ctypes.POINTER(DashShape)


def lib():
    """Load libdash.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    L.dash_abi_version.restype = _I
    L.dash_abi_version.argtypes = []
    L.dash_status_string.restype = ctypes.c_char_p
    L.dash_status_string.argtypes = [_I]
    L.dash_workspace_size.restype = _SZ
    L.dash_workspace_size.argtypes = [_I, _SHAPE]
    L.dash_get_layout.restype = _I
    L.dash_get_layout.argtypes = [_SHAPE, _I, ctypes.POINTER(DashLayout)]
    L.dash_summarize.restype = _I
    L.dash_summarize.argtypes = [_SHAPE, _P, _P, _P, _P, _SZ, _P]
    L.dash_route.restype = _I
    L.dash_summarize_diagonal.restype = _I
    L.dash_summarize_diagonal.argtypes = [_SHAPE, _P, _P, _P, _P]
    L.dash_route.argtypes = [_SHAPE, _P, _P, _P, _F, _P, _F, _F, _F, _I, _P, _P, _P, _P, _SZ,
                             _P]
    L.dash_attn_prefill.restype = _I
    L.dash_attn_prefill.argtypes = [_SHAPE, _P, _P, _P, _P, _F, _P, _F, _F, _F, _I, _I, _P,
                                    _P, _P, _P, _SZ, _P]
    L.dash_attn_sparse.restype = _I
    L.dash_attn_sparse.argtypes = [_SHAPE, _P, _P, _P, _P, _P, _F, _I, _P, _P, _P, _SZ, _P]
    L.dash_attn_decode.restype = _I
    L.dash_attn_decode.argtypes = [_SHAPE, _P, _P, _P, _P, _P, _P, _F, _F, _F, _F, _I, _I, _P,
                                   _P, _P, _P, _SZ, _P]
    L.dash_attn_decode_append.restype = _I
    L.dash_attn_decode_append.argtypes = [_SHAPE, _P, _P, _P, _P, _P, _P, _P, _P, _F, _F, _F,
                                          _F, _I, _I, _P, _P, _P, _P, _SZ, _P]
    L.dash_attn_decode_noalloc.restype = _I
    L.dash_attn_decode_noalloc.argtypes = [_SHAPE, _P, _P, _P, _P, _P, _P, _F, _F, _F, _F, _I,
                                           _I, _P, _P, _P, _P]
    L.dash_prefill_schedule.restype = _I
    L.dash_prefill_schedule.argtypes = [_SHAPE, _I, _P, _SZ, ctypes.POINTER(ctypes.c_int), _P]
    L.dash_probe_peak.restype = _I
    L.dash_probe_peak.argtypes = [_I, _P, _SZ, _I, _P, _SZ, ctypes.POINTER(ctypes.c_double), _P]
    L.dash_noalloc_scratch_need.restype = _SZ
    L.dash_noalloc_scratch_need.argtypes = [_SHAPE]
    L.dash_route_topk.restype = _I
    L.dash_route_topk.argtypes = [_SHAPE, _P, _P, _I, _F, _F, _I, _P, _P, _P, _P, _SZ, _P]
    L.dash_attn_decode_sparse.restype = _I
    L.dash_attn_decode_sparse.argtypes = [_SHAPE, _P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _P,
                                          _SZ, _P]
    L.dash_attn_sparse_backward.restype = _I
    L.dash_attn_sparse_backward.argtypes = [_SHAPE, _P, _P, _P, _P, _P, _P, _P, _P, _F, _I,
                                            _P, _P, _P, _P, _P, _SZ, _P]
    L.dash_attn_prefill_backward.restype = _I
    L.dash_attn_prefill_backward.argtypes = [_SHAPE, _P, _P, _P, _P, _F, _P, _F, _F, _F, _I,
                                             _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
    L.dash_cache_append.restype = _I
    L.dash_cache_append.argtypes = [_SHAPE, _P, _P, _P, _P, _P, _P, _P, _P]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().dash_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != DASH_OK:
        raise DashError(fn, status, status_string(status))


def make_shape(num_seqs, max_seqlen, total_tokens, cu_seqlens_ptr, Hq, Hkv, D, B, dtype):
    return DashShape(int(num_seqs), int(max_seqlen), int(total_tokens),
                     cu_seqlens_ptr if cu_seqlens_ptr else None, int(Hq), int(Hkv), int(D),
                     int(B), int(dtype))


def layout(shape: DashShape, enable_gqa: bool = True) -> DashLayout:
    out = DashLayout()
    check("dash_get_layout", lib().dash_get_layout(ctypes.byref(shape), int(enable_gqa),
                                                   ctypes.byref(out)))
    return out


def workspace_size(op: int, shape: DashShape) -> int:
    return int(lib().dash_workspace_size(op, ctypes.byref(shape)))

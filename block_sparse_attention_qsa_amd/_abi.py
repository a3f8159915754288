"""ctypes declarations of the C ABI in include/qsa.h: the batch struct and
every entry point's signature.  Plain ctypes (no torch), so that a process
can drive the library's host-side ABI layer on its own."""
from __future__ import annotations

import ctypes


class CBatch(ctypes.Structure):
    """qsa_batch."""
    _fields_ = [("num_req", ctypes.c_int32), ("num_q", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("q_start", ctypes.c_void_p), ("seq_len", ctypes.c_void_p), ("kv_start", ctypes.c_void_p),
                ("blk_start", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("pages_per_req", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float

SIGNATURES = {
    "qsa_abi_version": (ctypes.c_int, []),
    "qsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qsa_workspace_bytes": (_SZ, [_P, _I32, _I32, _I32]),
    "qsa_score": (ctypes.c_int, [_P, _P, _P, _P, _I64, _P]),
    "qsa_select_topk": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _P, _P, _SZ, _P]),
    "qsa_build_index": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, _P]),
    "qsa_select_positions": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "qsa_sparse_attn": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _P, _P, _I32, _F, _P, _I32,
                                       _P, _SZ, _P]),
    "qsa_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _F, _P, _I32,
                                  _P, _P, _P, _P, _P, _SZ, _P]),
    "qsa_compress_keys": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "qsa_decode_static": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _F, _P, _I32,
                                         _P, _P, _P, _P, _P]),
    "qsa_debug_build": (ctypes.c_int, []),
    "qsa_error_read": (ctypes.c_int, [_P, _I32]),
}


def load(path: str) -> ctypes.CDLL:
    """Load a build of the library and declare every entry point's types."""
    handle = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle

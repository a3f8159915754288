"""QSA block-sparse decode attention on MI355X (gfx950).

Thin Python binding of libqsa.so (C ABI in include/qsa.h).  Each function
here marshals torch tensors to device pointers and the current HIP stream and
calls the entry point of the same name; every step of the computation runs in
the library's HIP kernels.  PyTorch provides device memory and streams only.

There is no fallback: if the library is not built, or a call fails, a
QsaError is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["QsaError", "Batch", "lib", "abi_version", "status_string", "workspace_bytes", "alloc_workspace",
           "qsa_score", "qsa_select_topk", "qsa_build_index", "qsa_sparse_attn", "qsa_decode", "qsa_compress_keys",
           "qsa_decode_static", "qsa_select_positions", "STATIC_SCRATCH_BYTES", "use_library", "debug_build", "error_read",
           "ERROR_BAD_QUERIES", "ERROR_BAD_PAGE", "ERROR_BAD_POSITIONS", "ERROR_BAD_BLOCKS",
           "ERROR_BAD_SELECTION",
           "BLOCK", "TOPK", "WIDTH", "INDEX_DIM", "HEAD_DIM", "KV_BF16", "KV_FP8_E4M3", "OUT_F32", "OUT_BF16"]

BLOCK = 4
TOPK = 512
WIDTH = BLOCK * TOPK + BLOCK - 1
INDEX_DIM = 128
HEAD_DIM = 128
KV_BF16, KV_FP8_E4M3 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
STATIC_SCRATCH_BYTES = 64 << 20
ERROR_BAD_QUERIES, ERROR_BAD_PAGE, ERROR_BAD_POSITIONS, ERROR_BAD_BLOCKS, ERROR_BAD_SELECTION = 0x1, 0x2, 0x4, 0x8, 0x10

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libqsa_debug.so")   # device-side precondition checks


class QsaError(RuntimeError):
    pass


from ._abi import CBatch as _CBatch, load as _load_abi   # noqa: E402

_lib = None


_use_debug = os.environ.get("QSA_DEBUG_LIBRARY", "") not in ("", "0")
_handles = {}


def use_library(debug: bool) -> None:
    """Route every following call to libqsa_debug.so (debug=True: the same
    kernels with device-side precondition checks reported in the error word)
    or to libqsa.so."""
    global _lib, _use_debug
    _use_debug = bool(debug)
    _lib = None


def lib() -> ctypes.CDLL:
    """Load libqsa.so, or libqsa_debug.so after use_library(True) (both built
    in-tree by block_sparse_attention_qsa_amd.build)."""
    global _lib
    if _lib is None:
        path = DEBUG_LIB_PATH if _use_debug else LIB_PATH
        if path in _handles:
            _lib = _handles[path]
            return _lib
        if not os.path.exists(path):
            raise QsaError(f"{path} is not built; run `python -m block_sparse_attention_qsa_amd.build`")
        handle = _load_abi(path)
        _handles[path] = handle
        _lib = handle
    return _lib


def debug_build() -> bool:
    return bool(lib().qsa_debug_build())


def error_read(clear: bool = False) -> int:
    """The current device's error word (QSA_ERROR_* bits set by kernels since
    it was last cleared); synchronises with the device."""
    bits = ctypes.c_uint32(0)
    _check(lib().qsa_error_read(ctypes.byref(bits), int(clear)), "qsa_error_read")
    return int(bits.value)


def abi_version() -> int:
    return lib().qsa_abi_version()


def status_string(status: int) -> str:
    return lib().qsa_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise QsaError(f"{what}: {status_string(status)} (status {status})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtypes, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise QsaError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise QsaError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise QsaError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise QsaError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_FP8 = (torch.float8_e4m3fn, torch.uint8)


class Batch:
    """Batch metadata: per-request query ranges, lengths and cache offsets.

    Host arrays (numpy / CPU tensors / lists) are copied to `device` and the
    host scalars (num_req, num_q, max_blocks) derived from them.  Device int32
    tensors are used as they are and then num_q and max_blocks must be given.
    A paged KV cache is described by page_table ([num_req, pages_per_req]
    int32, physical page of each logical page) and page_size (a multiple of
    4); kv_start is then unused and may be None.
    """

    def __init__(self, q_start, seq_len, kv_start, blk_start, *, num_q: Optional[int] = None,
                 max_blocks: Optional[int] = None, page_table=None, page_size: Optional[int] = None,
                 device="cuda"):
        def to_dev(x):
            if isinstance(x, torch.Tensor) and x.is_cuda:
                if x.dtype != torch.int32 or not x.is_contiguous():
                    raise QsaError("device metadata must be contiguous int32")
                return x
            return torch.as_tensor(x, dtype=torch.int32).contiguous().to(device)

        host = not (isinstance(seq_len, torch.Tensor) and seq_len.is_cuda)
        if host:
            qs = [int(v) for v in (q_start.tolist() if hasattr(q_start, "tolist") else q_start)]
            sl = [int(v) for v in (seq_len.tolist() if hasattr(seq_len, "tolist") else seq_len)]
            num_q = qs[-1] if num_q is None else num_q
            max_blocks = max(s // BLOCK for s in sl) if max_blocks is None else max_blocks
        if num_q is None or max_blocks is None:
            raise QsaError("num_q and max_blocks are required with device metadata")
        self.q_start = to_dev(q_start)
        self.seq_len = to_dev(seq_len)
        self.kv_start = None if kv_start is None else to_dev(kv_start)
        self.blk_start = to_dev(blk_start)
        self.num_req = int(self.seq_len.shape[0])
        self.num_q = int(num_q)
        self.max_blocks = int(max_blocks)
        self.page_table = None
        self.page_size = 0
        pages_per_req = 0
        if page_table is not None:
            if page_size is None:
                raise QsaError("page_size is required with a page table")
            self.page_table = to_dev(page_table)
            if self.page_table.dim() != 2 or self.page_table.shape[0] != self.num_req:
                raise QsaError("page_table must be [num_req, pages_per_req]")
            self.page_size = int(page_size)
            pages_per_req = int(self.page_table.shape[1])
        elif self.kv_start is None:
            raise QsaError("kv_start is required without a page table")
        ptr = lambda t: None if t is None else t.data_ptr()
        self._c = _CBatch(self.num_req, self.num_q, self.max_blocks, ptr(self.q_start), ptr(self.seq_len),
                          ptr(self.kv_start), ptr(self.blk_start), ptr(self.page_table), self.page_size,
                          pages_per_req)

    @property
    def c(self):
        return ctypes.byref(self._c)


def workspace_bytes(batch: Batch, num_q_heads: int, num_kv_heads: int, k: int = TOPK) -> int:
    return int(lib().qsa_workspace_bytes(batch.c, num_q_heads, num_kv_heads, k))


def alloc_workspace(batch: Batch, num_q_heads: int, num_kv_heads: int, k: int = TOPK,
                    device="cuda") -> torch.Tensor:
    """A zero-filled workspace of the size the library asks for (the library
    keeps it zeroed between calls)."""
    n = workspace_bytes(batch, num_q_heads, num_kv_heads, k)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def qsa_score(batch: Batch, idx_q, ckeys, scores, stream=None) -> None:
    _dev(idx_q, "idx_q", _BF16, (batch.num_q, INDEX_DIM))
    _dev(ckeys, "ckeys", _BF16)
    if ckeys.dim() != 2 or ckeys.shape[1] != INDEX_DIM:
        raise QsaError("ckeys must be [rows, 128]")
    _dev(scores, "scores", (torch.float32,))
    if scores.dim() != 2 or scores.shape[0] != batch.num_q:
        raise QsaError("scores must be [num_q, ld]")
    _check(lib().qsa_score(batch.c, _ptr(idx_q), _ptr(ckeys), _ptr(scores), scores.shape[1], _stream(stream)),
           "qsa_score")


def qsa_select_topk(batch: Batch, scores, sel, n_sel, k: int = TOPK, workspace=None, stream=None) -> None:
    """Rows longer than 32,768 blocks need workspace; without one, a
    workspace of qsa_workspace_bytes() is allocated for the call."""
    _dev(scores, "scores", (torch.float32,))
    if scores.dim() != 2 or scores.shape[0] != batch.num_q:
        raise QsaError("scores must be [num_q, ld]")
    _dev(sel, "sel", (torch.int32,), (batch.num_q, k))
    _dev(n_sel, "n_sel", (torch.int32,), (batch.num_q,))
    if workspace is None:
        workspace = alloc_workspace(batch, 1, 1, k, device=scores.device)
    ws_n = workspace.numel() * workspace.element_size()
    _check(lib().qsa_select_topk(batch.c, _ptr(scores), scores.shape[1], k, _ptr(sel), _ptr(n_sel),
                                 _ptr(workspace), ws_n, _stream(stream)), "qsa_select_topk")


def qsa_select_positions(batch: Batch, scores, sel, n_sel, pos, n_pos, k: int = TOPK, workspace=None,
                         stream=None) -> None:
    """Selection and position buffer in one launch (as qsa_decode runs them)."""
    _dev(scores, "scores", (torch.float32,))
    if scores.dim() != 2 or scores.shape[0] != batch.num_q:
        raise QsaError("scores must be [num_q, ld]")
    _dev(sel, "sel", (torch.int32,), (batch.num_q, k))
    _dev(n_sel, "n_sel", (torch.int32,), (batch.num_q,))
    _dev(pos, "pos", (torch.int32,), (batch.num_q, BLOCK * k + BLOCK - 1))
    _dev(n_pos, "n_pos", (torch.int32,), (batch.num_q,))
    if workspace is None:
        workspace = alloc_workspace(batch, 1, 1, k, device=scores.device)
    ws_n = workspace.numel() * workspace.element_size()
    _check(lib().qsa_select_positions(batch.c, _ptr(scores), scores.shape[1], k, _ptr(sel), _ptr(n_sel), _ptr(pos),
                                      _ptr(n_pos), _ptr(workspace), ws_n, _stream(stream)), "qsa_select_positions")


def qsa_build_index(batch: Batch, sel, n_sel, pos, n_pos, k: int = TOPK, stream=None) -> None:
    _dev(sel, "sel", (torch.int32,), (batch.num_q, k))
    _dev(n_sel, "n_sel", (torch.int32,), (batch.num_q,))
    _dev(pos, "pos", (torch.int32,), (batch.num_q, BLOCK * k + BLOCK - 1))
    _dev(n_pos, "n_pos", (torch.int32,), (batch.num_q,))
    _check(lib().qsa_build_index(batch.c, _ptr(sel), _ptr(n_sel), k, _ptr(pos), _ptr(n_pos), _stream(stream)),
           "qsa_build_index")


def _kv_args(k_cache, v_cache, k_scale, v_scale, num_kv_heads):
    if k_cache.dtype in _FP8:
        kv = KV_FP8_E4M3
        _dev(k_cache, "k_cache", _FP8)
        _dev(v_cache, "v_cache", _FP8)
        _dev(k_scale, "k_scale", (torch.float32,), (num_kv_heads,))
        _dev(v_scale, "v_scale", (torch.float32,), (num_kv_heads,))
    else:
        kv = KV_BF16
        _dev(k_cache, "k_cache", _BF16)
        _dev(v_cache, "v_cache", _BF16)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dim() != 3 or t.shape[1] != num_kv_heads or t.shape[2] != HEAD_DIM:
            raise QsaError(f"{name} must be [slots, {num_kv_heads}, {HEAD_DIM}]")
    return kv


def _out_dtype(out) -> int:
    if out.dtype == torch.float32:
        return OUT_F32
    if out.dtype == torch.bfloat16:
        return OUT_BF16
    raise QsaError("out must be float32 or bfloat16")


def qsa_sparse_attn(batch: Batch, q, k_cache, v_cache, pos, n_pos, out, *, k_scale=None, v_scale=None,
                    sm_scale: Optional[float] = None, workspace=None, stream=None) -> None:
    if q.dim() != 3 or q.shape[0] != batch.num_q or q.shape[2] != HEAD_DIM:
        raise QsaError("q must be [num_q, Hq, 128]")
    hq, hkv = int(q.shape[1]), int(k_cache.shape[1])
    _dev(q, "q", _BF16)
    kv = _kv_args(k_cache, v_cache, k_scale, v_scale, hkv)
    _dev(pos, "pos", (torch.int32,))
    if pos.dim() != 2 or pos.shape[0] != batch.num_q:
        raise QsaError("pos must be [num_q, width]")
    _dev(n_pos, "n_pos", (torch.int32,), (batch.num_q,))
    _dev(out, "out", (torch.float32, torch.bfloat16), (batch.num_q, hq, HEAD_DIM))
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else float(sm_scale)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qsa_sparse_attn(batch.c, _ptr(q), _ptr(k_cache), _ptr(v_cache), kv, _ptr(k_scale), _ptr(v_scale),
                                 hq, hkv, _ptr(pos), _ptr(n_pos), pos.shape[1], sm, _ptr(out), _out_dtype(out),
                                 _ptr(workspace), ws_n, _stream(stream)), "qsa_sparse_attn")


def qsa_decode(batch: Batch, idx_q, ckeys, q, k_cache, v_cache, out, workspace, *, k_scale=None, v_scale=None,
               k: int = TOPK, sm_scale: Optional[float] = None, sel=None, n_sel=None, pos=None, n_pos=None,
               stream=None) -> None:
    _dev(idx_q, "idx_q", _BF16, (batch.num_q, INDEX_DIM))
    _dev(ckeys, "ckeys", _BF16)
    if ckeys.dim() != 2 or ckeys.shape[1] != INDEX_DIM:
        raise QsaError("ckeys must be [rows, 128]")
    if q.dim() != 3 or q.shape[0] != batch.num_q or q.shape[2] != HEAD_DIM:
        raise QsaError("q must be [num_q, Hq, 128]")
    hq, hkv = int(q.shape[1]), int(k_cache.shape[1])
    _dev(q, "q", _BF16)
    kv = _kv_args(k_cache, v_cache, k_scale, v_scale, hkv)
    _dev(out, "out", (torch.float32, torch.bfloat16), (batch.num_q, hq, HEAD_DIM))
    width = BLOCK * k + BLOCK - 1
    if sel is not None:
        _dev(sel, "sel", (torch.int32,), (batch.num_q, k))
    if n_sel is not None:
        _dev(n_sel, "n_sel", (torch.int32,), (batch.num_q,))
    if pos is not None:
        _dev(pos, "pos", (torch.int32,), (batch.num_q, width))
    if n_pos is not None:
        _dev(n_pos, "n_pos", (torch.int32,), (batch.num_q,))
    _dev(workspace, "workspace", (torch.uint8,))
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else float(sm_scale)
    _check(lib().qsa_decode(batch.c, _ptr(idx_q), _ptr(ckeys), _ptr(q), _ptr(k_cache), _ptr(v_cache), kv,
                            _ptr(k_scale), _ptr(v_scale), hq, hkv, k, sm, _ptr(out), _out_dtype(out),
                            _ptr(sel), _ptr(n_sel), _ptr(pos), _ptr(n_pos), _ptr(workspace),
                            workspace.numel(), _stream(stream)), "qsa_decode")


def qsa_decode_static(batch: Batch, idx_q, ckeys, q, k_cache, v_cache, out, *, k_scale=None, v_scale=None,
                      k: int = TOPK, sm_scale: Optional[float] = None, sel=None, n_sel=None, pos=None, n_pos=None,
                      stream=None) -> None:
    """qsa_decode on the library's own per-device scratch (no workspace
    argument; see qsa.h for its size limit and sharing rules)."""
    _dev(idx_q, "idx_q", _BF16, (batch.num_q, INDEX_DIM))
    _dev(ckeys, "ckeys", _BF16)
    if ckeys.dim() != 2 or ckeys.shape[1] != INDEX_DIM:
        raise QsaError("ckeys must be [rows, 128]")
    if q.dim() != 3 or q.shape[0] != batch.num_q or q.shape[2] != HEAD_DIM:
        raise QsaError("q must be [num_q, Hq, 128]")
    hq, hkv = int(q.shape[1]), int(k_cache.shape[1])
    _dev(q, "q", _BF16)
    kv = _kv_args(k_cache, v_cache, k_scale, v_scale, hkv)
    _dev(out, "out", (torch.float32, torch.bfloat16), (batch.num_q, hq, HEAD_DIM))
    width = BLOCK * k + BLOCK - 1
    for name, t, shape in (("sel", sel, (batch.num_q, k)), ("n_sel", n_sel, (batch.num_q,)),
                           ("pos", pos, (batch.num_q, width)), ("n_pos", n_pos, (batch.num_q,))):
        if t is not None:
            _dev(t, name, (torch.int32,), shape)
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else float(sm_scale)
    _check(lib().qsa_decode_static(batch.c, _ptr(idx_q), _ptr(ckeys), _ptr(q), _ptr(k_cache), _ptr(v_cache), kv,
                                   _ptr(k_scale), _ptr(v_scale), hq, hkv, k, sm, _ptr(out), _out_dtype(out),
                                   _ptr(sel), _ptr(n_sel), _ptr(pos), _ptr(n_pos), _stream(stream)),
           "qsa_decode_static")


def qsa_compress_keys(batch: Batch, prev_len, tok_keys, ckeys, stream=None) -> None:
    """Compressed keys of the blocks completed since prev_len (see qsa.h)."""
    _dev(prev_len, "prev_len", (torch.int32,), (batch.num_req,))
    _dev(tok_keys, "tok_keys", _BF16)
    _dev(ckeys, "ckeys", _BF16)
    for name, t in (("tok_keys", tok_keys), ("ckeys", ckeys)):
        if t.dim() != 2 or t.shape[1] != INDEX_DIM:
            raise QsaError(f"{name} must be [rows, {INDEX_DIM}]")
    _check(lib().qsa_compress_keys(batch.c, _ptr(prev_len), _ptr(tok_keys), _ptr(ckeys), _stream(stream)),
           "qsa_compress_keys")

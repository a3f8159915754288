"""The C-ABI library loads, exports every entry point include/qsa.h declares,
and rejects bad host arguments before enqueuing anything (no GPU needed: none
of these calls reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_qsa_amd as qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(qsa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_five_stage_calls():
    names = declared_functions()
    for n in ("qsa_score", "qsa_select_topk", "qsa_build_index", "qsa_sparse_attn", "qsa_decode",
              "qsa_workspace_bytes", "qsa_status_string", "qsa_abi_version", "qsa_compress_keys"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = qsa.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert qsa.abi_version() == 2
    for s in range(6):
        assert qsa.status_string(s)
    assert qsa.status_string(99) == "unknown status"


def _cbatch(num_req=1, num_q=4, max_blocks=12500, ptr=0x1000, page_table=None, page_size=0, pages=0):
    return qsa._CBatch(num_req, num_q, max_blocks, ptr, ptr, ptr, ptr, page_table, page_size, pages)


def test_workspace_bytes_host_only():
    lib = qsa.lib()
    b = _cbatch()
    n = lib.qsa_workspace_bytes(ctypes.byref(b), 32, 4, 512)
    # at least: scores + sel + pos for 4 queries
    assert n >= 4 * 12500 * 4 + 4 * 512 * 4 + 4 * 2051 * 4
    assert n % 256 == 0
    assert lib.qsa_workspace_bytes(ctypes.byref(b), 32, 3, 512) == 0      # Hq % Hkv != 0
    assert lib.qsa_workspace_bytes(ctypes.byref(b), 32, 4, 513) == 0      # k > 512
    assert lib.qsa_workspace_bytes(None, 32, 4, 512) == 0


def test_error_paths_return_before_launch():
    lib = qsa.lib()
    P = ctypes.c_void_p(0x1000)
    good = _cbatch()
    assert lib.qsa_score(None, P, P, P, 12500, None) == 1
    assert lib.qsa_score(ctypes.byref(good), None, P, P, 12500, None) == 1
    assert lib.qsa_score(ctypes.byref(good), P, P, P, 100, None) == 2          # ld < max_blocks
    assert lib.qsa_score(ctypes.byref(good), P, P, P, (1 << 26) + 1, None) == 2  # ld past 2^26
    bad_q = _cbatch(num_req=1, num_q=5)
    assert lib.qsa_score(ctypes.byref(bad_q), P, P, P, 12500, None) == 2       # > 4 queries per request
    nullmeta = qsa._CBatch(1, 1, 10, 0, 0, 0, 0, 0, 0, 0)
    assert lib.qsa_score(ctypes.byref(nullmeta), P, P, P, 10, None) == 1
    # paged batches: page size a positive multiple of 4, at least one page per request;
    # kv_start may then be NULL
    assert lib.qsa_score(ctypes.byref(_cbatch(page_table=0x1000, page_size=6, pages=4)), P, P, P, 12500, None) == 2
    assert lib.qsa_score(ctypes.byref(_cbatch(page_table=0x1000, page_size=16, pages=0)), P, P, P, 12500, None) == 2
    assert lib.qsa_score(ctypes.byref(_cbatch(page_table=0x1000, page_size=0, pages=4)), P, P, P, 12500, None) == 2
    nokv = qsa._CBatch(1, 4, 12500, 0x1000, 0x1000, 0, 0x1000, 0, 0, 0)
    assert lib.qsa_build_index(ctypes.byref(nokv), P, P, 512, P, P, None) == 1
    assert lib.qsa_compress_keys(ctypes.byref(good), None, P, P, None) == 1
    assert lib.qsa_compress_keys(ctypes.byref(bad_q), P, P, P, None) == 2
    assert lib.qsa_select_topk(ctypes.byref(good), P, 12500, 0, P, P, None, 0, None) == 2
    assert lib.qsa_build_index(ctypes.byref(good), P, P, 600, P, P, None) == 2
    # attention: bad head geometry / dtype / scale / width / workspace
    args = lambda hq, hkv, kvd, ks, width, sm, odt, ws, wsn: lib.qsa_sparse_attn(
        ctypes.byref(good), P, P, P, kvd, ks, ks, hq, hkv, P, P, width, sm, P, odt, ws, wsn, None)
    assert args(32, 3, 0, None, 2051, 0.08, 0, P, 1 << 30) == 2
    assert args(64, 2, 0, None, 2051, 0.08, 0, P, 1 << 30) == 3              # group of 32 > 16
    assert args(32, 4, 7, None, 2051, 0.08, 0, P, 1 << 30) == 3
    assert args(32, 4, 1, None, 2051, 0.08, 0, P, 1 << 30) == 1              # FP8 without scales
    assert args(32, 4, 0, None, 2050, 0.08, 0, P, 1 << 30) == 2              # width not 4k+3
    assert args(32, 4, 0, None, 2051, -1.0, 0, P, 1 << 30) == 2
    assert args(32, 4, 0, None, 2051, 0.08, 2, P, 1 << 30) == 3
    assert args(32, 4, 0, None, 2051, 0.08, 0, None, 0) == 4                 # workspace needed
    assert args(32, 4, 0, None, 2051, 0.08, 0, ctypes.c_void_p(0x1004), 1 << 30) == 4   # misaligned
    # output alignment: 16 bytes for FP32, 8 for BF16
    att_out = lambda out, odt: lib.qsa_sparse_attn(ctypes.byref(good), P, P, P, 0, None, None, 32, 4, P, P, 2051,
                                                   0.08, out, odt, P, 1 << 30, None)
    assert att_out(ctypes.c_void_p(0x1008), 0) == 2
    assert att_out(ctypes.c_void_p(0x1004), 1) == 2
    d = lambda ws, wsn: lib.qsa_decode(ctypes.byref(good), P, P, P, P, P, 0, None, None, 32, 4, 512, 0.08, P, 0,
                                       None, None, None, None, ws, wsn, None)
    assert d(P, 16) == 4
    assert d(None, 0) == 4


def test_python_binding_refuses_host_tensors():
    import torch
    b = qsa.Batch.__new__(qsa.Batch)
    with pytest.raises(qsa.QsaError):
        qsa._dev(torch.zeros(4, 128, dtype=torch.bfloat16), "idx_q", qsa._BF16)


def test_stream_probe_library_loads_and_checks_arguments():
    """The benchmark's stream-read probe (its roofline context, not part of
    the QSA ABI) is built beside the library and refuses bad arguments before
    launching."""
    from block_sparse_attention_qsa_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        pytest.fail(f"{PROBE_LIB} is not built; run the package build")
    probe = ctypes.CDLL(PROBE_LIB)
    fn = probe.qsa_probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert fn(None, 1 << 20, ctypes.c_void_p(0x1000), 4096, None) != 0              # no source
    assert fn(ctypes.c_void_p(0x1004), 1 << 20, ctypes.c_void_p(0x1000), 4096, None) != 0   # misaligned
    assert fn(ctypes.c_void_p(0x1000), 1 << 20, ctypes.c_void_p(0x1000), 0, None) != 0     # no grid

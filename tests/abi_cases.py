"""Host-side checks of the C ABI that need no GPU: every call here is
rejected by argument validation before anything is enqueued, or only sizes a
workspace.  Plain ctypes, so the same checks run against the release library
(test_abi.py) and against a build whose host code runs under AddressSanitizer
(abi_asan_driver.py)."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")
P = ctypes.c_void_p(0x1000)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(qsa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def cbatch(CBatch, num_req=1, num_q=4, max_blocks=12500, ptr=0x1000, page_table=None, page_size=0, pages=0):
    return CBatch(num_req, num_q, max_blocks, ptr, ptr, ptr, ptr, page_table, page_size, pages)


def check_exports(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def check_version_and_strings(lib):
    assert lib.qsa_abi_version() == 2
    for s in range(7):
        assert lib.qsa_status_string(s)
    assert lib.qsa_status_string(99) == b"unknown status"
    assert lib.qsa_status_string(-1) == b"unknown status"


def check_workspace_sizes(lib, CBatch):
    b = cbatch(CBatch)
    n = lib.qsa_workspace_bytes(ctypes.byref(b), 32, 4, 512)
    # at least: the 128 KiB control region, then scores + sel + pos for 4 queries
    assert n >= 128 * 1024 + 4 * 12500 * 4 + 4 * 512 * 4 + 4 * 2051 * 4
    assert n % 256 == 0
    assert lib.qsa_workspace_bytes(ctypes.byref(b), 32, 3, 512) == 0      # Hq % Hkv != 0
    assert lib.qsa_workspace_bytes(ctypes.byref(b), 32, 4, 513) == 0      # k > 512
    assert lib.qsa_workspace_bytes(None, 32, 4, 512) == 0
    for num_req, num_q, mb in ((1, 1, 0), (1, 1, 1), (32, 128, 15300), (64, 256, 32768), (1, 4, 1 << 20),
                               (16384, 65536, 8)):
        bb = cbatch(CBatch, num_req=num_req, num_q=num_q, max_blocks=mb)
        for hq, hkv in ((16, 2), (32, 4), (4, 4), (64, 4)):
            for k in (1, 100, 512):
                got = lib.qsa_workspace_bytes(ctypes.byref(bb), hq, hkv, k)
                assert got >= 128 * 1024 and got % 256 == 0


def check_error_paths(lib, CBatch):
    good = cbatch(CBatch)
    assert lib.qsa_score(None, P, P, P, 12500, None) == 1
    assert lib.qsa_score(ctypes.byref(good), None, P, P, 12500, None) == 1
    assert lib.qsa_score(ctypes.byref(good), P, P, P, 100, None) == 2          # ld < max_blocks
    assert lib.qsa_score(ctypes.byref(good), P, P, P, (1 << 26) + 1, None) == 2  # ld past 2^26
    bad_q = cbatch(CBatch, num_req=1, num_q=5)
    assert lib.qsa_score(ctypes.byref(bad_q), P, P, P, 12500, None) == 2       # > 4 queries per request
    assert lib.qsa_score(ctypes.byref(cbatch(CBatch, num_req=0, num_q=0)), P, P, P, 12500, None) == 2
    assert lib.qsa_score(ctypes.byref(cbatch(CBatch, max_blocks=(1 << 20) + 1)), P, P, P, 1 << 21, None) == 2
    nullmeta = CBatch(1, 1, 10, 0, 0, 0, 0, 0, 0, 0)
    assert lib.qsa_score(ctypes.byref(nullmeta), P, P, P, 10, None) == 1
    # paged batches: page size a positive multiple of 4, at least one page per request;
    # kv_start may then be NULL
    pt = 0x1000
    assert lib.qsa_score(ctypes.byref(cbatch(CBatch, page_table=pt, page_size=6, pages=4)), P, P, P, 12500, None) == 2
    assert lib.qsa_score(ctypes.byref(cbatch(CBatch, page_table=pt, page_size=16, pages=0)), P, P, P, 12500, None) == 2
    assert lib.qsa_score(ctypes.byref(cbatch(CBatch, page_table=pt, page_size=0, pages=4)), P, P, P, 12500, None) == 2
    assert lib.qsa_score(ctypes.byref(cbatch(CBatch, page_table=pt, page_size=1 << 20, pages=1 << 12)),
                         P, P, P, 12500, None) == 2                              # page_size * pages past int32
    nokv = CBatch(1, 4, 12500, 0x1000, 0x1000, 0, 0x1000, 0, 0, 0)
    assert lib.qsa_build_index(ctypes.byref(nokv), P, P, 512, P, P, None) == 1
    assert lib.qsa_compress_keys(ctypes.byref(good), None, P, P, None) == 1
    assert lib.qsa_compress_keys(ctypes.byref(bad_q), P, P, P, None) == 2
    assert lib.qsa_select_topk(ctypes.byref(good), P, 12500, 0, P, P, None, 0, None) == 2
    assert lib.qsa_select_topk(ctypes.byref(good), None, 12500, 512, P, P, None, 0, None) == 1
    long_rows = cbatch(CBatch, max_blocks=40000)
    assert lib.qsa_select_topk(ctypes.byref(long_rows), P, 40000, 512, P, P, None, 0, None) == 4   # needs workspace
    assert lib.qsa_select_topk(ctypes.byref(long_rows), P, 40000, 512, P, P, P, 1024, None) == 4
    assert lib.qsa_build_index(ctypes.byref(good), P, P, 600, P, P, None) == 2
    assert lib.qsa_select_positions(ctypes.byref(good), P, 12500, 512, P, P, None, P, None, 0, None) == 1
    assert lib.qsa_select_positions(ctypes.byref(good), P, 100, 512, P, P, P, P, None, 0, None) == 2
    assert lib.qsa_select_positions(ctypes.byref(long_rows), P, 40000, 512, P, P, P, P, None, 0, None) == 4
    # attention: bad head geometry / dtype / scale / width / workspace
    args = lambda hq, hkv, kvd, ks, width, sm, odt, ws, wsn: lib.qsa_sparse_attn(
        ctypes.byref(good), P, P, P, kvd, ks, ks, hq, hkv, P, P, width, sm, P, odt, ws, wsn, None)
    assert args(32, 3, 0, None, 2051, 0.08, 0, P, 1 << 30) == 2
    assert args(64, 2, 0, None, 2051, 0.08, 0, P, 1 << 30) == 3              # group of 32 > 16
    assert args(32, 4, 7, None, 2051, 0.08, 0, P, 1 << 30) == 3
    assert args(32, 4, 1, None, 2051, 0.08, 0, P, 1 << 30) == 1              # FP8 without scales
    assert args(32, 4, 0, None, 2050, 0.08, 0, P, 1 << 30) == 2              # width not 4k+3
    assert args(32, 4, 0, None, 2055, 0.08, 0, P, 1 << 30) == 2              # width past 2,051
    assert args(32, 4, 0, None, 2051, -1.0, 0, P, 1 << 30) == 2
    assert args(32, 4, 0, None, 2051, float("nan"), 0, P, 1 << 30) == 2
    assert args(32, 4, 0, None, 2051, 0.08, 2, P, 1 << 30) == 3
    assert args(32, 4, 0, None, 2051, 0.08, 0, None, 0) == 4                 # workspace needed (split units)
    assert args(32, 4, 0, None, 2051, 0.08, 0, ctypes.c_void_p(0x1004), 1 << 30) == 4   # misaligned
    assert args(32, 4, 0, None, 2051, 0.08, 0, P, 4096) == 4                 # too small
    # a batch of several requests writes the attention's work list to the
    # workspace even when no unit is split (k = 1: one 32-position chunk)
    two = cbatch(CBatch, num_req=2, num_q=4, max_blocks=8)
    rag = lambda ws, wsn: lib.qsa_sparse_attn(ctypes.byref(two), P, P, P, 0, None, None, 32, 4, P, P, 7, 0.08, P, 0,
                                              ws, wsn, None)
    assert rag(None, 0) == 4
    assert rag(P, 128 * 1024) == 4
    # output alignment: 16 bytes for FP32, 8 for BF16
    att_out = lambda out, odt: lib.qsa_sparse_attn(ctypes.byref(good), P, P, P, 0, None, None, 32, 4, P, P, 2051,
                                                   0.08, out, odt, P, 1 << 30, None)
    assert att_out(ctypes.c_void_p(0x1008), 0) == 2
    assert att_out(ctypes.c_void_p(0x1004), 1) == 2
    d = lambda ws, wsn: lib.qsa_decode(ctypes.byref(good), P, P, P, P, P, 0, None, None, 32, 4, 512, 0.08, P, 0,
                                       None, None, None, None, ws, wsn, None)
    assert d(P, 16) == 4
    assert d(None, 0) == 4
    assert lib.qsa_decode(ctypes.byref(good), None, P, P, P, P, 0, None, None, 32, 4, 512, 0.08, P, 0,
                          None, None, None, None, P, 1 << 30, None) == 1
    # the allocation-free decode: a batch past its scratch is refused before any device call
    huge = CBatch(64, 256, 1 << 20, 0x1000, 0x1000, 0x1000, 0x1000, None, 0, 0)
    assert lib.qsa_workspace_bytes(ctypes.byref(huge), 32, 4, 512) > 64 << 20
    assert lib.qsa_decode_static(ctypes.byref(huge), P, P, P, P, P, 0, None, None, 32, 4, 512, 0.088, P, 0,
                                 None, None, None, None, None) == 6
    assert lib.qsa_decode_static(ctypes.byref(good), P, P, P, P, P, 0, None, None, 32, 3, 512, 0.088, P, 0,
                                 None, None, None, None, None) == 2
    # diagnostics
    assert lib.qsa_error_read(None, 0) == 1


def run_all(lib, CBatch):
    check_exports(lib)
    check_version_and_strings(lib)
    check_workspace_sizes(lib, CBatch)
    check_error_paths(lib, CBatch)

"""The C-ABI library loads, exports every entry point include/qsa.h declares,
and rejects bad host arguments before enqueuing anything (no GPU needed: none
of these calls reaches a kernel launch)."""
import ctypes
import os

import pytest

import abi_cases
import block_sparse_attention_qsa_amd as qsa


def test_header_declares_the_five_stage_calls():
    names = abi_cases.declared_functions()
    for n in ("qsa_score", "qsa_select_topk", "qsa_build_index", "qsa_sparse_attn", "qsa_decode",
              "qsa_workspace_bytes", "qsa_status_string", "qsa_abi_version", "qsa_compress_keys",
              "qsa_decode_static", "qsa_error_read", "qsa_debug_build"):
        assert n in names


def test_library_exports_every_declared_symbol():
    abi_cases.check_exports(qsa.lib())


def test_version_and_status_strings():
    abi_cases.check_version_and_strings(qsa.lib())


def test_workspace_bytes_host_only():
    abi_cases.check_workspace_sizes(qsa.lib(), qsa._CBatch)


def test_error_paths_return_before_launch():
    abi_cases.check_error_paths(qsa.lib(), qsa._CBatch)


def test_debug_library_exports_the_same_abi():
    from block_sparse_attention_qsa_amd.build import DEBUG_LIB
    if not os.path.exists(DEBUG_LIB):
        pytest.fail(f"{DEBUG_LIB} is not built; run the package build")
    from block_sparse_attention_qsa_amd._abi import load
    dbg = load(DEBUG_LIB)
    abi_cases.run_all(dbg, qsa._CBatch)
    assert dbg.qsa_debug_build() == 1
    assert qsa.lib().qsa_debug_build() == 0


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

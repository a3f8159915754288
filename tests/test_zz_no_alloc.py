"""qsa_decode_static (the entry point that allocates nothing and keeps its
scratch in the library's own per-device array) against qsa_decode on the same
inputs: two calls in a row, the second on a smaller batch, each checked for
equal selections, positions and output bits, and against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_qsa_amd as qsa
from workloads import make_custom, make_workload
from workloads.device import upload
from gpu_helpers import (SM_SCALE, assert_out_close, assert_selection_equal, batch_of, need_gpu, oracle_decode,
                         run_decode, say)

pytestmark = pytest.mark.gpu


def _static_decode(w, dev):
    b = batch_of(w)
    k = qsa.TOPK
    out = torch.full((w.num_q, w.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((w.num_q, k), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((w.num_q,), -7, dtype=torch.int32, device="cuda")
    pos = torch.full((w.num_q, 4 * k + 3), -7, dtype=torch.int32, device="cuda")
    n_pos = torch.full((w.num_q,), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_decode_static(b, dev["idx_q"], dev["ckeys"], dev["q"], dev["k_cache"], dev["v_cache"], out,
                          k_scale=dev["k_scale"], v_scale=dev["v_scale"], sm_scale=SM_SCALE, sel=sel, n_sel=n_sel,
                          pos=pos, n_pos=n_pos)
    torch.cuda.synchronize()
    return {"out": out.cpu().numpy().astype(np.float64), "sel": sel.cpu().numpy(), "n_sel": n_sel.cpu().numpy(),
            "pos": pos.cpu().numpy(), "n_pos": n_pos.cpu().numpy()}


def test_static_decode_matches_workspace_decode():
    need_gpu()
    big = make_workload("mtp50k")
    small = make_custom("static-small", [8192, 37, 3001], [1, 4, 2], 16, 2, kv_dtype="fp8_e4m3", seed=77)
    for w in (big, small):          # the second call is on a smaller batch
        say("qsa_decode_static", w.name, "queries", w.num_q)
        dev = upload(w)
        got = _static_decode(w, dev)
        ref_call = run_decode(w, dev)
        assert_selection_equal(got, ref_call)
        assert np.array_equal(got["out"].view(np.uint64), ref_call["out"].view(np.uint64))
        ref = oracle_decode(w, want_scores=False)
        assert_selection_equal(got, ref)
        assert_out_close(got["out"], ref["out"])
        # and the production form (no debug outputs) of the static call
        lean = torch.empty((w.num_q, w.num_q_heads, 128), dtype=torch.float32, device="cuda")
        qsa.qsa_decode_static(batch_of(w), dev["idx_q"], dev["ckeys"], dev["q"], dev["k_cache"], dev["v_cache"],
                              lean, k_scale=dev["k_scale"], v_scale=dev["v_scale"], sm_scale=SM_SCALE)
        torch.cuda.synchronize()
        assert np.array_equal(lean.cpu().numpy().astype(np.float64).view(np.uint64), got["out"].view(np.uint64))


def test_static_decode_rejects_batches_past_its_scratch():
    """A batch whose workspace would exceed the static scratch is refused
    before anything is enqueued (host check; the pointers are never used)."""
    lib = qsa.lib()
    P = ctypes.c_void_p(0x1000)
    huge = qsa._CBatch(64, 256, 1 << 20, 0x1000, 0x1000, 0x1000, 0x1000, None, 0, 0)
    assert lib.qsa_workspace_bytes(ctypes.byref(huge), 32, 4, 512) > qsa.STATIC_SCRATCH_BYTES
    st = lib.qsa_decode_static(ctypes.byref(huge), P, P, P, P, P, 0, None, None, 32, 4, 512, 0.088, P, 0,
                               None, None, None, None, None)
    assert st == 6, st

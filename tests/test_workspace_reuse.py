"""One zero-filled workspace, sized for the largest batch, serves calls of
different batch geometry in turn (a serving loop whose batch changes every
step): the 8K single-query decode, the 50K batch-1 MTP verify step and the
32-request FP8 batch, then the first two again.  Every call is checked
against the oracle (selection and positions bit-exact, output within
2e-3 * max|out|), and the workspace's control region is zero after each."""
import gc

import numpy as np
import pytest
import torch

import block_sparse_attention_qsa_amd as qsa
from workloads import make_workload
from workloads.device import upload
from gpu_helpers import (SM_SCALE, assert_out_close, assert_selection_equal, batch_of, need_gpu, oracle_decode,
                         run_decode, say)

pytestmark = pytest.mark.gpu

CTL_BYTES = 128 * 1024
ORDER = ["single8k", "mtp50k", "mtp50k_b32_fp8", "single8k", "mtp50k"]


def test_decode_one_workspace_across_geometries():
    need_gpu()
    names = sorted(set(ORDER))
    ws_bytes = {}
    for n in names:
        w = make_workload(n)
        ws_bytes[n] = qsa.workspace_bytes(batch_of(w), w.num_q_heads, w.num_kv_heads)
    ws = torch.zeros(max(ws_bytes.values()), dtype=torch.uint8, device="cuda")
    say("workspace bytes", ws_bytes, "shared", ws.numel())
    refs = {}
    for n in ORDER:
        w = make_workload(n)
        if n not in refs:
            say("oracle", n)
            refs[n] = oracle_decode(w, want_scores=False)
        say("qsa_decode on the shared workspace", n)
        dev = upload(w)
        got = run_decode(w, dev, ws=ws)
        assert_selection_equal(got, refs[n])
        assert_out_close(got["out"], refs[n]["out"])
        # the production call (no debug outputs) on the same workspace
        lean = run_decode(w, dev, ws=ws, debug=False)
        assert np.array_equal(lean["out"].view(np.uint64), got["out"].view(np.uint64))
        assert int(ws[:CTL_BYTES].sum().item()) == 0
        del dev, got, lean
        gc.collect()
        torch.cuda.empty_cache()


def test_sparse_attn_one_workspace_across_geometries():
    """The stage call qsa_sparse_attn alone, alternating geometries whose split
    counts and partial sizes differ, on one workspace."""
    need_gpu()
    order = ["mtp50k", "single8k", "mtp50k", "single8k"]
    ws = None
    refs = {}
    for n in order:
        w = make_workload(n)
        b = batch_of(w)
        if ws is None:
            ws = torch.zeros(max(qsa.workspace_bytes(batch_of(make_workload(m)), make_workload(m).num_q_heads,
                                                     make_workload(m).num_kv_heads) for m in set(order)),
                             dtype=torch.uint8, device="cuda")
        if n not in refs:
            refs[n] = oracle_decode(w, want_scores=False)
        ref = refs[n]
        dev = upload(w)
        out = torch.full((w.num_q, w.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
        say("qsa_sparse_attn on the shared workspace", n)
        qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], torch.from_numpy(ref["pos"]).cuda(),
                            torch.from_numpy(ref["n_pos"]).cuda(), out, k_scale=dev["k_scale"],
                            v_scale=dev["v_scale"], sm_scale=SM_SCALE, workspace=ws)
        torch.cuda.synchronize()
        assert_out_close(out.cpu().numpy().astype(np.float64), ref["out"])
        assert int(ws[:CTL_BYTES].sum().item()) == 0


def test_long_row_select_between_decodes_on_one_workspace():
    """The stage selector keeps long rows' slice candidates in the workspace
    after its control region, so a qsa_select_topk call between two decode
    calls on the same workspace disturbs no counter the decode relies on."""
    import oracle
    need_gpu()
    w = make_workload("mtp50k")
    b = batch_of(w)
    nfs = [140001, 90000, 70001, 33000]
    rng = np.random.default_rng(1201)
    rows = [rng.integers(-300, 300, n).astype(np.float32) for n in nfs]
    lb = qsa.Batch([0, 1, 2, 3, 4], [4 * n for n in nfs], [0, 0, 0, 0], [0, 0, 0, 0])
    S = torch.zeros((4, max(nfs)), dtype=torch.float32, device="cuda")
    for i, r in enumerate(rows):
        S[i, :len(r)] = torch.from_numpy(r).cuda()
    ws = torch.zeros(max(qsa.workspace_bytes(b, w.num_q_heads, w.num_kv_heads), qsa.workspace_bytes(lb, 1, 1)),
                     dtype=torch.uint8, device="cuda")
    ref = oracle_decode(w, want_scores=False)
    dev = upload(w)
    for rep in range(2):
        got = run_decode(w, dev, ws=ws)
        assert_selection_equal(got, ref)
        assert_out_close(got["out"], ref["out"])
        sel = torch.full((4, qsa.TOPK), -7, dtype=torch.int32, device="cuda")
        n_sel = torch.full((4,), -7, dtype=torch.int32, device="cuda")
        say("qsa_select_topk long rows on the shared workspace", rep)
        qsa.qsa_select_topk(lb, S, sel, n_sel, workspace=ws)
        torch.cuda.synchronize()
        for i, r in enumerate(rows):
            exp = oracle.select_blocks(r.astype(np.float64), qsa.TOPK)
            assert np.array_equal(sel[i].cpu().numpy()[:len(exp)], exp), i
        assert int(ws[:CTL_BYTES].sum().item()) == 0

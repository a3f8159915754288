"""The debug build (libqsa_debug.so, compiled with QSA_DEBUG_CHECKS) checks the
device-side preconditions that release builds trust and reports a breach in
the per-device error word instead of clamping silently.  Each case here feeds
one breach that the kernels' own clamps keep inside the buffers (so nothing
faults): a token past the request's page-table row, a request with five
queries, a position buffer that breaks the 4-slot run rule, a selection count
past k, and a row longer than max_blocks.  Valid inputs leave the word at 0
and give the release library's bits; the release library reports nothing."""
import numpy as np
import pytest
import torch

import block_sparse_attention_qsa_amd as qsa
from workloads import make_custom, paged_layout
from workloads.device import upload
from gpu_helpers import SM_SCALE, batch_of, decode_paged, need_gpu, run_decode, say

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_lib():
    need_gpu()
    qsa.use_library(True)
    assert qsa.debug_build()
    qsa.error_read(clear=True)
    yield
    qsa.error_read(clear=True)
    qsa.use_library(False)


def _paged(w, page_size, seed):
    """BF16 workload re-laid out in pages (see paged_layout)."""
    table, kc, vc = paged_layout(w, page_size, seed)
    dev = upload(w)
    for name, c in (("k_cache", kc), ("v_cache", vc)):
        dev[name] = torch.from_numpy(np.ascontiguousarray(c).view(np.int16)).cuda().view(torch.bfloat16)
    return table, dev


def test_valid_inputs_report_nothing_and_match_release(debug_lib):
    w = make_custom("dbg-valid", [6001, 2050, 37, 9000], [4, 2, 1, 3], 16, 2, kv_dtype="fp8_e4m3", seed=1301)
    dev = upload(w)
    got = run_decode(w, dev)
    assert qsa.error_read(clear=True) == 0
    qsa.use_library(False)
    rel = run_decode(w, dev)
    qsa.use_library(True)
    assert np.array_equal(got["pos"], rel["pos"])
    assert np.array_equal(got["out"].view(np.uint64), rel["out"].view(np.uint64))


def test_valid_paged_long_row_and_stage_calls_report_nothing(debug_lib):
    """Valid inputs on the paths the first case does not take: a paged cache
    with a row past 32,768 blocks (two-step selection, positions through the
    page table; the stage index builder runs inside decode_paged too) and the
    stage attention over positions in permuted runs.  The word stays 0 and the
    bits equal the release library's."""
    w = make_custom("dbg-valid-long", [140000, 57, 3001], [4, 1, 2], 16, 2, kv_dtype="fp8_e4m3", seed=1310)
    say("debug build: valid paged long row")
    got = decode_paged(w, 64, 1311)[0]
    assert qsa.error_read(clear=True) == 0
    dev = upload(w)
    b = batch_of(w)
    rng = np.random.default_rng(1312)
    dbg = run_decode(w, dev)
    pos = dbg["pos"].copy()
    for qi in range(w.num_q):          # the kept blocks' 4-slot runs in another order
        full = int(dbg["n_pos"][qi]) // 4
        order = rng.permutation(full)
        pos[qi, :4 * full] = pos[qi, :4 * full].reshape(full, 4)[order].reshape(-1)
    outs = []
    for debug in (True, False):
        qsa.use_library(debug)
        out = torch.full((w.num_q, 16, 128), float("nan"), dtype=torch.float32, device="cuda")
        ws = qsa.alloc_workspace(b, 16, 2)
        qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], torch.from_numpy(pos).cuda(),
                            torch.from_numpy(dbg["n_pos"]).cuda(), out, k_scale=dev["k_scale"],
                            v_scale=dev["v_scale"], sm_scale=SM_SCALE, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        assert qsa.error_read(clear=True) == 0
    qsa.use_library(False)
    rel = decode_paged(w, 64, 1311)[0]
    qsa.use_library(True)
    assert np.array_equal(got["pos"], rel["pos"])
    assert np.array_equal(got["out"].view(np.uint64), rel["out"].view(np.uint64))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_page_past_the_table_row(debug_lib):
    w = make_custom("dbg-page", [3000, 1200], [4, 2], 16, 2, seed=1302)
    table, dev = _paged(w, 64, seed=1303)
    # the table keeps only the pages of the first 2,048 tokens of each request:
    # later tokens' logical pages run past the row (the kernels clamp them)
    short = np.ascontiguousarray(table[:, :2048 // 64])
    b = qsa.Batch(w.q_start, w.seq_len, None, w.blk_start, page_table=short, page_size=64)
    out = torch.empty((w.num_q, 16, 128), dtype=torch.float32, device="cuda")
    ws = qsa.alloc_workspace(b, 16, 2)
    say("debug build: page past the row")
    qsa.qsa_decode(b, dev["idx_q"], dev["ckeys"], dev["q"], dev["k_cache"], dev["v_cache"], out, ws, sm_scale=SM_SCALE)
    bits = qsa.error_read(clear=True)
    assert bits & qsa.ERROR_BAD_PAGE, bits
    # the release library runs the same call without a report
    qsa.use_library(False)
    qsa.qsa_decode(b, dev["idx_q"], dev["ckeys"], dev["q"], dev["k_cache"], dev["v_cache"], out, ws, sm_scale=SM_SCALE)
    assert qsa.error_read(clear=True) == 0
    qsa.use_library(True)


def test_five_queries_in_one_request(debug_lib):
    w = make_custom("dbg-nq", [5000, 800], [4, 2], 16, 2, seed=1304)
    dev = upload(w)
    # request 0 claims 5 of the 6 queries (the host check only bounds the total)
    b = qsa.Batch(np.array([0, 5, 6]), w.seq_len, w.kv_start, w.blk_start)
    out = torch.empty((w.num_q, 16, 128), dtype=torch.float32, device="cuda")
    ws = qsa.alloc_workspace(b, 16, 2)
    say("debug build: five queries in a request")
    qsa.qsa_decode(b, dev["idx_q"], dev["ckeys"], dev["q"], dev["k_cache"], dev["v_cache"], out, ws, sm_scale=SM_SCALE)
    assert qsa.error_read(clear=True) & qsa.ERROR_BAD_QUERIES


def test_position_buffer_breaking_the_run_rule(debug_lib):
    w = make_custom("dbg-pos", [9000], [4], 16, 2, seed=1305)
    dev = upload(w)
    b = batch_of(w)
    sel = torch.empty((w.num_q, qsa.TOPK), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.num_q,), dtype=torch.int32, device="cuda")
    pos = torch.empty((w.num_q, qsa.WIDTH), dtype=torch.int32, device="cuda")
    n_pos = torch.empty((w.num_q,), dtype=torch.int32, device="cuda")
    ws = qsa.alloc_workspace(b, 16, 2)
    out = torch.empty((w.num_q, 16, 128), dtype=torch.float32, device="cuda")
    qsa.qsa_decode(b, dev["idx_q"], dev["ckeys"], dev["q"], dev["k_cache"], dev["v_cache"], out, ws,
                   sm_scale=SM_SCALE, sel=sel, n_sel=n_sel, pos=pos, n_pos=n_pos)
    assert qsa.error_read(clear=True) == 0
    bad = pos.clone()
    bad[0, 5], bad[0, 6] = pos[0, 6], pos[0, 5]          # two slots of one run swapped: still valid slots
    say("debug build: broken position runs")
    qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], bad, n_pos, out, sm_scale=SM_SCALE, workspace=ws)
    assert qsa.error_read(clear=True) & qsa.ERROR_BAD_POSITIONS
    long_n = n_pos.clone()
    long_n[1] = qsa.WIDTH + 7                             # past the buffer: the kernel clamps it to the width
    qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], pos, long_n, out, sm_scale=SM_SCALE, workspace=ws)
    assert qsa.error_read(clear=True) & qsa.ERROR_BAD_POSITIONS


def test_selection_count_past_k_and_unsorted(debug_lib):
    w = make_custom("dbg-sel", [9000, 4000], [2, 1], 16, 2, seed=1306)
    b = batch_of(w)
    sel = torch.arange(qsa.TOPK, dtype=torch.int32, device="cuda").repeat(w.num_q, 1).contiguous()
    n_sel = torch.full((w.num_q,), qsa.TOPK, dtype=torch.int32, device="cuda")
    pos = torch.empty((w.num_q, qsa.WIDTH), dtype=torch.int32, device="cuda")
    n_pos = torch.empty((w.num_q,), dtype=torch.int32, device="cuda")
    qsa.qsa_build_index(b, sel, n_sel, pos, n_pos)
    assert qsa.error_read(clear=True) == 0
    n_sel[0] = qsa.TOPK + 1
    qsa.qsa_build_index(b, sel, n_sel, pos, n_pos)
    assert qsa.error_read(clear=True) & qsa.ERROR_BAD_SELECTION
    n_sel[0] = qsa.TOPK
    sel[1, 10] = 3                                        # not ascending
    qsa.qsa_build_index(b, sel, n_sel, pos, n_pos)
    assert qsa.error_read(clear=True) & qsa.ERROR_BAD_SELECTION


def test_row_longer_than_max_blocks(debug_lib):
    w = make_custom("dbg-blocks", [9000], [1], 16, 2, seed=1307)
    dev = upload(w)
    b = qsa.Batch(w.q_start, w.seq_len, w.kv_start, w.blk_start, max_blocks=1000)   # 2,250 blocks in the row
    scores = torch.zeros((w.num_q, 1000), dtype=torch.float32, device="cuda")
    qsa.qsa_score(b, dev["idx_q"], dev["ckeys"], scores)
    assert qsa.error_read(clear=True) & qsa.ERROR_BAD_BLOCKS

"""Per-stage and fused parity of the HIP path against the CPU oracle on small
inputs that still span several tiles, workgroups and ragged tails."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_qsa_amd as qsa
import oracle
from workloads import make_custom
from workloads.device import upload
from gpu_helpers import (SM_SCALE, assert_lean_decode_same, assert_out_close, assert_selection_equal, batch_of, need_gpu, oracle_decode,
                         run_decode, say)

pytestmark = pytest.mark.gpu

CTL_BYTES = 128 * 1024     # the workspace's fixed control region (all counters)


def _mixed_workload(kv="bf16", index_values="int", hq=16, hkv=2, seed=201):
    lens = [1, 2, 3, 4, 5, 17, 300, 2051, 2055, 9000, 12345, 20000]
    nq = [1, 2, 3, 4, 1, 4, 2, 4, 3, 4, 1, 4]
    return make_custom(f"mixed-{kv}-{index_values}", lens, nq, hq, hkv, kv_dtype=kv, seed=seed,
                       index_values=index_values)


def test_score_bit_exact_integer_inputs():
    need_gpu()
    w = _mixed_workload()
    say("qsa_score", w.name)
    dev = upload(w)
    b = batch_of(w)
    ld = b.max_blocks + 5
    scores = torch.full((w.num_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_score(b, dev["idx_q"], dev["ckeys"], scores)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    for r in range(w.num_req):
        nblk = int(w.seq_len[r]) // 4
        b0 = int(w.blk_start[r])
        for qi in w.queries_of(r):
            ref = oracle.block_scores(w.idx_q[qi], w.ckeys[b0:b0 + nblk])
            assert np.array_equal(s[qi, :nblk].view(np.uint32), ref.view(np.uint32)), (r, qi)
            assert np.all(np.isnan(s[qi, nblk:])), "wrote past the request's blocks"


def test_score_normal_inputs_close():
    need_gpu()
    w = _mixed_workload(index_values="normal")
    say("qsa_score normal", w.name)
    dev = upload(w)
    b = batch_of(w)
    scores = torch.zeros((w.num_q, b.max_blocks), dtype=torch.float32, device="cuda")
    qsa.qsa_score(b, dev["idx_q"], dev["ckeys"], scores)
    torch.cuda.synchronize()
    s = scores.cpu().numpy().astype(np.float64)
    for r in range(w.num_req):
        nblk = int(w.seq_len[r]) // 4
        b0 = int(w.blk_start[r])
        keys = oracle.bf16_to_f64(w.ckeys[b0:b0 + nblk])
        for qi in w.queries_of(r):
            iq = oracle.bf16_to_f64(w.idx_q[qi])
            ref = oracle.block_scores(w.idx_q[qi], w.ckeys[b0:b0 + nblk]).astype(np.float64)
            bound = 128 * 2.0 ** -23 * (np.abs(keys) @ np.abs(iq)) + 1e-30
            assert np.all(np.abs(s[qi, :nblk] - ref) <= bound), (r, qi)


def _select_case(nfs, kind, seed):
    """One query per request with exactly nf full blocks and given score style."""
    rng = np.random.default_rng(seed)
    rows = []
    for nf in nfs:
        if kind == "ties":
            s = rng.integers(-4, 5, nf).astype(np.float32)
        elif kind == "normal":
            s = rng.standard_normal(nf).astype(np.float32)
        elif kind == "zeros":
            s = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), nf)
        elif kind == "wide":
            s = (rng.standard_normal(nf) * 10.0 ** rng.integers(-30, 30, nf)).astype(np.float32)
        elif kind == "inf":
            # infinite scores leave the row without a finite range: the
            # selector falls back to radix passes over the raw keys
            s = rng.standard_normal(nf).astype(np.float32)
            s[rng.random(nf) < 0.01] = np.inf
            s[rng.random(nf) < 0.01] = -np.inf
        elif kind == "spiky":
            # a flat row with a few hundred high outliers: the value range is
            # set by the outliers, so almost the whole row shares the lowest
            # few grid bins and every outlier is kept
            s = (rng.standard_normal(nf) * 0.01).astype(np.float32)
            hot = rng.choice(nf, min(nf, 300), replace=False)
            s[hot] = rng.integers(10, 21, len(hot)).astype(np.float32)
        elif kind == "flat":
            # 60% of the blocks share the top score: the chosen top-level radix
            # bin can exceed what the selector stages in LDS
            s = rng.uniform(-3.0, 2.0, nf).astype(np.float32)
            s[rng.random(nf) < 0.6] = 2.5
        else:
            raise ValueError(kind)
        rows.append(s)
    return rows


SELECT_GROUPS = {
    # one launch per group: the largest row decides which selector variant runs
    "le16k": [0, 1, 511, 512, 513, 1000, 2048, 12500, 16383, 16384],
    # the segment width follows the longest row: 10, 12 and 14 scores per thread
    "e10": [1, 513, 9000, 10240],
    "e12": [7, 10241, 12288],
    "e14": [12289, 12500, 14336],
    "le32k": [3, 513, 4097, 16385, 20000, 32768],
    "le64k": [600, 32769, 40000, 65535, 65536],
    "stream": [700, 12500, 65537, 100000, 131072],
    "ms262k": [5, 32769, 131073, 262144],
    # the longest row the library takes (QSA_MAX_BLOCKS: a 4M-token context)
    "max4m": [1 << 20, 70001],
}


@pytest.mark.parametrize("group", list(SELECT_GROUPS))
@pytest.mark.parametrize("kind", ["ties", "normal", "zeros", "wide", "flat", "inf", "spiky"])
def test_select_bit_exact(kind, group):
    need_gpu()
    nfs = SELECT_GROUPS[group]
    rows = _select_case(nfs, kind, seed=301 + len(kind) + 7 * len(group))
    say("qsa_select_topk", kind, group, nfs)
    B = len(nfs)
    seq = [4 * nf + (i % 4) for i, nf in enumerate(nfs)]
    seq = [max(s, 1) for s in seq]
    b = qsa.Batch(np.arange(B + 1), seq, np.zeros(B), np.zeros(B))
    ld = b.max_blocks + (3 if kind in ("ties", "wide") else 0)    # unaligned rows too
    S = np.zeros((B, ld), np.float32)
    for i, s in enumerate(rows):
        S[i, :len(s)] = s
    scores = torch.from_numpy(S).cuda()
    sel = torch.full((B, 512), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_select_topk(b, scores, sel, n_sel)
    torch.cuda.synchronize()
    sel, n_sel = sel.cpu().numpy(), n_sel.cpu().numpy()
    for i, s in enumerate(rows):
        ref = oracle.select_blocks(s, 512)
        assert n_sel[i] == len(ref), (i, nfs[i])
        assert np.array_equal(sel[i, :len(ref)], ref), (i, nfs[i])
        assert np.all(sel[i, len(ref):] == -1)


@pytest.mark.parametrize("k", [1, 7, 64, 512])
def test_select_small_k(k):
    need_gpu()
    nfs = [3, 64, 65, 700, 5000]
    rows = _select_case(nfs, "ties", seed=400 + k)
    say("qsa_select_topk k", k)
    B = len(nfs)
    b = qsa.Batch(np.arange(B + 1), [4 * nf for nf in nfs], np.zeros(B), np.zeros(B))
    S = np.zeros((B, b.max_blocks), np.float32)
    for i, s in enumerate(rows):
        S[i, :len(s)] = s
    sel = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_select_topk(b, torch.from_numpy(S).cuda(), sel, n_sel, k=k)
    torch.cuda.synchronize()
    sel, n_sel = sel.cpu().numpy(), n_sel.cpu().numpy()
    for i, s in enumerate(rows):
        ref = oracle.select_blocks(s, k)
        assert n_sel[i] == len(ref)
        assert np.array_equal(sel[i, :len(ref)], ref)



@pytest.mark.parametrize("nf", [700, 12500, 20000, 70000])
def test_select_nan_scores(nf):
    """NaN scores (finite keys and queries never produce them) leave a valid
    selection.  The positive quiet NaN sorts above +Inf, so a row holding a few
    of them selects as the oracle does with +Inf in their place (no row here
    holds an Inf).  Where a negative NaN sorts is not fixed, so that row is
    checked for what holds either way: k distinct ascending blocks of the row
    that include the oracle's top k - m of the row without its m NaNs.  NaNs
    sit in full waves (no grid bin: their histogram count goes to a guard
    word) and in the last one."""
    need_gpu()
    rng = np.random.default_rng(4242 + nf)
    k = 512
    base = rng.standard_normal((2, nf)).astype(np.float32)
    at = np.unique(np.concatenate([[0, 5, 63, nf // 2, nf - 1], rng.choice(nf, 20, replace=False)]))
    pos_nan = np.array([0x7FC00000], np.uint32).view(np.float32)[0]
    neg_nan = np.array([0xFFC00000], np.uint32).view(np.float32)[0]
    rows = base.copy()
    rows[0, at] = pos_nan
    rows[1, at] = neg_nan
    say("qsa_select_topk NaN rows", nf, "NaNs", len(at))
    b = qsa.Batch(np.arange(3), [4 * nf, 4 * nf], np.zeros(2), np.zeros(2))
    sel = torch.full((2, k), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_select_topk(b, torch.from_numpy(rows).cuda(), sel, n_sel)
    torch.cuda.synchronize()
    sel, n_sel = sel.cpu().numpy(), n_sel.cpu().numpy()
    as_inf = base[0].copy()
    as_inf[at] = np.inf
    ref = oracle.select_blocks(as_inf, k)
    assert n_sel[0] == k and np.array_equal(sel[0], ref)
    got = sel[1]
    assert n_sel[1] == k
    assert np.all(np.diff(got) > 0) and got[0] >= 0 and got[-1] < nf
    rest = np.delete(np.arange(nf), at)
    top = rest[oracle.select_blocks(base[1, rest], k - len(at))]
    assert np.all(np.isin(top, got))


@pytest.mark.parametrize("k", [1, 7, 100, 511])
@pytest.mark.parametrize("kind", ["ties", "normal"])
def test_select_small_k_long_rows(k, kind):
    """Rows past 32,768 blocks with k < 512: every slice keeps min(k, its
    blocks) candidates and the candidate rows are k per slice, so both slice
    sizes (8,192 blocks up to 262,144, 16,384 beyond) and a batch mixing long,
    short and tiny rows are checked against the oracle."""
    need_gpu()
    nfs = [300000, 70001, 40000, 32769, 5, 1000]
    rows = _select_case(nfs, kind, seed=500 + k + len(kind))
    say("qsa_select_topk long rows k", k, kind, nfs)
    for part in (nfs, nfs[1:]):          # longest row over / under 262,144 blocks
        off = len(nfs) - len(part)
        b = qsa.Batch(np.arange(len(part) + 1), [4 * nf + 1 for nf in part], np.zeros(len(part)),
                      np.zeros(len(part)))
        S = np.zeros((len(part), b.max_blocks), np.float32)
        for i in range(len(part)):
            S[i, :part[i]] = rows[off + i]
        sel = torch.full((len(part), k), -7, dtype=torch.int32, device="cuda")
        n_sel = torch.full((len(part),), -7, dtype=torch.int32, device="cuda")
        qsa.qsa_select_topk(b, torch.from_numpy(S).cuda(), sel, n_sel, k=k)
        torch.cuda.synchronize()
        sel_h, n_h = sel.cpu().numpy(), n_sel.cpu().numpy()
        for i in range(len(part)):
            ref = oracle.select_blocks(rows[off + i], k)
            assert n_h[i] == len(ref), (part[i], k)
            assert np.array_equal(sel_h[i, :len(ref)], ref), (part[i], k)
            assert np.all(sel_h[i, len(ref):] == -1)

@pytest.mark.parametrize("kind", ["ties", "normal"])
def test_select_long_rows_many_queries(kind):
    """A batch of 520 queries, three of them past 32,768 blocks (the two-step
    selector runs for the whole batch: every short row goes through the slice
    and candidate steps too), then its first 500 queries, on one workspace:
    every row checked against the oracle, the control region zero after
    each."""
    need_gpu()
    n = 520
    rng = np.random.default_rng(611 + len(kind))
    nfs = [int(x) for x in rng.integers(1, 3000, n)]
    nfs[7], nfs[300], nfs[499] = 40000, 70001, 33000          # rows past 32,768 blocks
    rows = _select_case(nfs, kind, seed=612 + len(kind))
    ws = None
    for part in (n, 500):
        b = qsa.Batch(np.arange(part + 1), [4 * nf + 1 for nf in nfs[:part]], np.zeros(part), np.zeros(part))
        if ws is None:
            ws = torch.zeros(qsa.workspace_bytes(b, 1, 1), dtype=torch.uint8, device="cuda")
        S = np.zeros((part, b.max_blocks), np.float32)
        for i in range(part):
            S[i, :nfs[i]] = rows[i]
        sel = torch.full((part, qsa.TOPK), -7, dtype=torch.int32, device="cuda")
        n_sel = torch.full((part,), -7, dtype=torch.int32, device="cuda")
        say("qsa_select_topk long rows, queries", part, kind)
        qsa.qsa_select_topk(b, torch.from_numpy(S).cuda(), sel, n_sel, workspace=ws)
        torch.cuda.synchronize()
        sel_h, n_h = sel.cpu().numpy(), n_sel.cpu().numpy()
        for i in range(part):
            ref = oracle.select_blocks(rows[i], qsa.TOPK)
            assert n_h[i] == len(ref), (part, i, nfs[i])
            assert np.array_equal(sel_h[i, :len(ref)], ref), (part, i, nfs[i])
            assert np.all(sel_h[i, len(ref):] == -1)
        assert int(ws[:CTL_BYTES].sum().item()) == 0


@pytest.mark.parametrize("lens,nq", [([1, 2, 3, 4, 5, 17, 300, 2051, 2055, 9000, 12345, 20000],
                                       [1, 2, 3, 4, 1, 4, 2, 4, 3, 4, 1, 4]),
                                      ([140001, 33000, 5000], [4, 2, 1])])
def test_select_positions_bit_exact(lens, nq):
    """Selection and positions from one launch (the stage form of what
    qsa_decode runs): both buffers bit-identical to the oracle's."""
    need_gpu()
    w = make_custom("selpos", lens, nq, 16, 2, seed=1401 + len(lens))
    ref = oracle_decode(w, want_scores=False)
    dev = upload(w)
    b = batch_of(w)
    scores = torch.zeros((w.num_q, b.max_blocks), dtype=torch.float32, device="cuda")
    qsa.qsa_score(b, dev["idx_q"], dev["ckeys"], scores)
    sel = torch.full((w.num_q, qsa.TOPK), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((w.num_q,), -7, dtype=torch.int32, device="cuda")
    pos = torch.full((w.num_q, qsa.WIDTH), -7, dtype=torch.int32, device="cuda")
    n_pos = torch.full((w.num_q,), -7, dtype=torch.int32, device="cuda")
    say("qsa_select_positions", w.name, max(lens))
    qsa.qsa_select_positions(b, scores, sel, n_sel, pos, n_pos)
    torch.cuda.synchronize()
    got = {"sel": sel.cpu().numpy(), "n_sel": n_sel.cpu().numpy(), "pos": pos.cpu().numpy(),
           "n_pos": n_pos.cpu().numpy()}
    assert_selection_equal(got, ref)


def test_build_index_bit_exact():
    need_gpu()
    w = _mixed_workload()
    say("qsa_build_index", w.name)
    ref = oracle_decode(w, want_scores=False)
    b = batch_of(w)
    sel = torch.from_numpy(ref["sel"]).cuda()
    n_sel = torch.from_numpy(ref["n_sel"]).cuda()
    pos = torch.full((w.num_q, 2051), -7, dtype=torch.int32, device="cuda")
    n_pos = torch.full((w.num_q,), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_build_index(b, sel, n_sel, pos, n_pos)
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), ref["pos"])
    assert np.array_equal(n_pos.cpu().numpy(), ref["n_pos"])


def test_binding_rejects_wrong_shapes():
    """The binding refuses device tensors of the wrong shape before any call
    into the library: position rows other than num_q, key rows other than 128
    wide."""
    need_gpu()
    w = make_custom("shapes", [3000, 700], [2, 1], 16, 2, seed=215)
    dev = upload(w)
    b = batch_of(w)
    out = torch.empty((w.num_q, 16, 128), dtype=torch.float32, device="cuda")
    ws = qsa.alloc_workspace(b, 16, 2)
    short_pos = torch.zeros((w.num_q - 1, qsa.WIDTH), dtype=torch.int32, device="cuda")
    n_pos = torch.ones((w.num_q,), dtype=torch.int32, device="cuda")
    with pytest.raises(qsa.QsaError, match="pos must be"):
        qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], short_pos, n_pos, out, sm_scale=SM_SCALE,
                            workspace=ws)
    flat_keys = dev["ckeys"].reshape(-1)
    for call in (lambda: qsa.qsa_decode(b, dev["idx_q"], flat_keys, dev["q"], dev["k_cache"], dev["v_cache"], out,
                                        ws, sm_scale=SM_SCALE),
                 lambda: qsa.qsa_decode_static(b, dev["idx_q"], flat_keys, dev["q"], dev["k_cache"],
                                               dev["v_cache"], out, sm_scale=SM_SCALE)):
        with pytest.raises(qsa.QsaError, match="ckeys must be"):
            call()


def test_decode_max_blocks():
    """The longest row the ABI takes: one request of 4,194,304 tokens, so its
    last verify query has 2^20 full blocks (QSA_MAX_BLOCKS) and the selection
    runs on 16,384-block slices and a 32,768-entry candidate row; FP8 KV."""
    need_gpu()
    w = make_custom("max-blocks", [4 * (1 << 20)], [4], 4, 1, kv_dtype="fp8_e4m3", seed=79, index_values="normal")
    assert int(w.seq_len[0]) // 4 == 1 << 20
    say("max blocks", int(w.seq_len[0]) // 4)
    ref = oracle_decode(w, want_scores=False)
    got = run_decode(w)
    assert_selection_equal(got, ref)
    assert_out_close(got["out"], ref["out"])


def test_decode_max_requests():
    """The largest batch the ABI takes: 16,384 requests (40,573 queries) of 1-64
    tokens, 24 of them long enough to need selection.  Grids reach 40,573
    workgroups and the request lookup its deepest search; a sample of queries
    (every query of the long rows, the first and last, and 300 others) is
    checked against the oracle."""
    need_gpu()
    rng = np.random.default_rng(77)
    R = 16384
    lens = rng.integers(1, 65, R)
    long_req = rng.choice(R, 24, replace=False)
    lens[long_req] = rng.integers(2100, 6000, 24)
    nq = np.minimum(rng.integers(1, 5, R), lens)
    w = make_custom("maxreq", lens.tolist(), nq.tolist(), 2, 1, kv_dtype="bf16", seed=78, index_values="normal")
    assert w.num_req == 16384          # QSA_MAX_REQUESTS
    say("max requests", w.num_req, "queries", w.num_q)
    got = run_decode(w)
    qs = set(int(x) for x in rng.choice(w.num_q, 300, replace=False)) | {0, w.num_q - 1}
    for r in long_req:
        qs |= set(range(int(w.q_start[r]), int(w.q_start[r + 1])))
    qs = sorted(qs)
    ref = oracle_decode(w, want_scores=False, queries=qs)
    assert_selection_equal(got, ref, queries=qs)
    assert_out_close(got["out"], ref["out"], queries=qs)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_ragged_batch_many_kv_heads(kv):
    """A batch of several requests whose (query, KV head) units stay under 512
    with 136 KV heads (GQA group 1), so the attention's work list carries KV
    head indices past 127: the fused decode (list written by the selection
    launch) and the stage attention (list from n_pos) against the oracle."""
    need_gpu()
    w = make_custom(f"heads136-{kv}", [600, 2100, 3001], [1, 1, 1], 136, 136, kv_dtype=kv, seed=209)
    say("ragged batch, 136 KV heads", kv)
    ref = oracle_decode(w, want_scores=False)
    dev = upload(w)
    got = run_decode(w, dev)
    assert_selection_equal(got, ref)
    assert_out_close(got["out"], ref["out"])
    assert_lean_decode_same(w, got, dev)
    b = batch_of(w)
    out = torch.full((w.num_q, w.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = qsa.alloc_workspace(b, w.num_q_heads, w.num_kv_heads)
    qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], torch.from_numpy(ref["pos"]).cuda(),
                        torch.from_numpy(ref["n_pos"]).cuda(), out, k_scale=dev["k_scale"], v_scale=dev["v_scale"],
                        sm_scale=SM_SCALE, workspace=ws)
    torch.cuda.synchronize()
    assert_out_close(out.cpu().numpy().astype(np.float64), ref["out"])


@pytest.mark.parametrize("k", [1, 7, 31])
def test_sparse_attn_small_k_several_requests(k):
    """Position rows of 4k + 3 <= 127 entries (one 32-position chunk step, so
    no unit is split) on a batch of several requests: the attention still
    follows the work list it lays out in the workspace, and the call without a
    workspace is refused before anything is enqueued."""
    need_gpu()
    w = _mixed_workload(kv="fp8_e4m3", hq=32, hkv=4, seed=207)
    say("qsa_sparse_attn small k", k, w.name)
    ref = oracle_decode(w, want_scores=False, k=k)
    dev = upload(w)
    b = batch_of(w)
    pos = torch.from_numpy(ref["pos"]).cuda()
    n_pos = torch.from_numpy(ref["n_pos"]).cuda()
    assert pos.shape[1] == 4 * k + 3
    out = torch.full((w.num_q, w.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(qsa.QsaError):
        qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], pos, n_pos, out, k_scale=dev["k_scale"],
                            v_scale=dev["v_scale"], sm_scale=SM_SCALE)
    ws = qsa.alloc_workspace(b, w.num_q_heads, w.num_kv_heads, k)
    for rep in range(2):
        qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], pos, n_pos, out, k_scale=dev["k_scale"],
                            v_scale=dev["v_scale"], sm_scale=SM_SCALE, workspace=ws)
        torch.cuda.synchronize()
        assert_out_close(out.cpu().numpy().astype(np.float64), ref["out"])
        assert int(ws[:128 * 1024].sum().item()) == 0


@pytest.mark.parametrize("kv,hq,hkv,out_dtype", [
    ("bf16", 16, 2, "f32"), ("fp8_e4m3", 16, 2, "f32"), ("bf16", 32, 4, "bf16"), ("fp8_e4m3", 32, 4, "bf16"),
    ("bf16", 4, 4, "f32"), ("bf16", 8, 2, "f32"), ("fp8_e4m3", 32, 2, "f32"), ("bf16", 12, 3, "f32"),
])
def test_sparse_attn_close(kv, hq, hkv, out_dtype):
    need_gpu()
    w = _mixed_workload(kv=kv, hq=hq, hkv=hkv, seed=500 + hq + hkv)
    say("qsa_sparse_attn", w.name, hq, hkv, out_dtype)
    ref = oracle_decode(w, want_scores=False)
    dev = upload(w)
    b = batch_of(w)
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = torch.full((w.num_q, hq, 128), float("nan"), dtype=tdt, device="cuda")
    ws = qsa.alloc_workspace(b, hq, hkv)
    pos = torch.from_numpy(ref["pos"]).cuda()
    n_pos = torch.from_numpy(ref["n_pos"]).cuda()
    for rep in range(2):     # the second call reuses the workspace the first left zeroed
        qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], pos, n_pos, out,
                            k_scale=dev["k_scale"], v_scale=dev["v_scale"], sm_scale=SM_SCALE, workspace=ws)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        if out_dtype == "f32":
            assert_out_close(got, ref["out"])
        else:
            # BF16 output: one extra rounding of at most 2^-8 relative on top of the FP32 bar
            r = ref["out"]
            err = np.abs(got - r) - 2.0 ** -8 * np.abs(r)
            assert err.max() <= 2e-3 * np.abs(r).max()


@pytest.mark.parametrize("hq,hkv,target_units,out_dtype", [(32, 4, 520, "f32"), (6, 3, 513, "bf16"), (8, 8, 512, "f32"),
                                                          (16, 2, 600, "f32")])
def test_sparse_attn_whole_units_fp8(hq, hkv, target_units, out_dtype):
    """FP8 batches with at least 512 (query, KV head) units, so no unit is
    split (the non-temporal, K-through-LDS kernel with its ping-pong
    buffers): even and odd unit counts, mixed lengths (a few blocks to past
    512 blocks, with partial blocks) and GQA groups of 8, 2 and 1, through
    the stage call and through the decode (with and without positions
    requested)."""
    need_gpu()
    rng = np.random.default_rng(900 + hq + hkv)
    lens, nq = [], []
    while sum(nq) * hkv < target_units:
        lens.append(int(rng.integers(5, 14000)))
        nq.append(int(rng.integers(1, 5)))
    if target_units % 2 != (sum(nq) * hkv) % 2:    # the odd case keeps an odd unit count
        lens.append(777)
        nq.append(1)
    w = make_custom(f"whole-{hq}-{hkv}", lens, nq, hq, hkv, kv_dtype="fp8_e4m3", seed=901 + hq)
    say("qsa_sparse_attn whole units", w.name, "queries", w.num_q, "units", w.num_q * hkv)
    assert w.num_q * hkv >= 512 and (w.num_q * hkv) % 2 == target_units % 2
    ref = oracle_decode(w, want_scores=False)
    dev = upload(w)
    b = batch_of(w)
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    ws = qsa.alloc_workspace(b, hq, hkv)

    def check(out):
        got = out.float().cpu().numpy().astype(np.float64)
        if out_dtype == "f32":
            assert_out_close(got, ref["out"])
        else:
            r = ref["out"]
            err = np.abs(got - r) - 2.0 ** -8 * np.abs(r)
            assert err.max() <= 2e-3 * np.abs(r).max()

    out = torch.full((w.num_q, hq, 128), float("nan"), dtype=tdt, device="cuda")
    qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], torch.from_numpy(ref["pos"]).cuda(),
                        torch.from_numpy(ref["n_pos"]).cuda(), out, k_scale=dev["k_scale"], v_scale=dev["v_scale"],
                        sm_scale=SM_SCALE, workspace=ws)
    torch.cuda.synchronize()
    check(out)
    if out_dtype == "f32":
        got = run_decode(w, dev, ws=ws)
        assert_selection_equal(got, ref)
        assert_out_close(got["out"], ref["out"])
        lean = run_decode(w, dev, ws=ws, debug=False)
        assert np.array_equal(lean["out"].view(np.uint64), got["out"].view(np.uint64))


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_sparse_attn_permuted_runs(kv):
    """A valid position buffer whose 4-slot runs come in a shuffled order (the
    partial block's run stays last, as the run rule requires): the output is
    the oracle's attention over the same rows."""
    need_gpu()
    w = _mixed_workload(kv=kv, seed=520)
    ref = oracle_decode(w, want_scores=False)
    rng = np.random.default_rng(521)
    pos = ref["pos"].copy()
    for qi in range(w.num_q):
        ns = (int(ref["n_pos"][qi]) // 4)            # full-block runs; the partial run stays at 4 * ns
        runs = pos[qi, :4 * ns].reshape(ns, 4)
        pos[qi, :4 * ns] = runs[rng.permutation(ns)].reshape(-1)
        # the shuffled buffer still obeys pos[i] = pos[i - i % 4] + i % 4
        i = np.arange(int(ref["n_pos"][qi]))
        assert np.array_equal(pos[qi, i], pos[qi, i - i % 4] + i % 4)
    assert not np.array_equal(pos, ref["pos"])
    dev = upload(w)
    b = batch_of(w)
    out = torch.full((w.num_q, w.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = qsa.alloc_workspace(b, w.num_q_heads, w.num_kv_heads)
    say("qsa_sparse_attn permuted runs", w.name)
    qsa.qsa_sparse_attn(b, dev["q"], dev["k_cache"], dev["v_cache"], torch.from_numpy(pos).cuda(),
                        torch.from_numpy(ref["n_pos"]).cuda(), out, k_scale=dev["k_scale"], v_scale=dev["v_scale"],
                        sm_scale=SM_SCALE, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    # the oracle over the same (permuted) rows, query by query
    for r in range(w.num_req):
        for qi in w.queries_of(r):
            rows = pos[qi, :int(ref["n_pos"][qi])]
            kr = oracle.qsa_oracle._dequant(w.k_cache, rows, w.kv_dtype, w.k_scale)
            vr = oracle.qsa_oracle._dequant(w.v_cache, rows, w.kv_dtype, w.v_scale)
            qh = oracle.bf16_to_f64(w.q[qi])
            exp = oracle.sparse_attention(qh, kr, vr, SM_SCALE)
            err = np.abs(got[qi] - exp).max() / np.abs(exp).max()
            assert err <= 2e-3, (qi, err)
    assert_out_close(got, ref["out"])


def test_decode_small_mixed():
    need_gpu()
    for kv in ("bf16", "fp8_e4m3"):
        w = _mixed_workload(kv=kv, seed=601)
        say("qsa_decode", w.name)
        ref = oracle_decode(w, want_scores=False)
        got = run_decode(w)
        assert_selection_equal(got, ref)
        assert_out_close(got["out"], ref["out"])
        assert_lean_decode_same(w, got)
        # every counter sits in the fixed control region at the start of the
        # workspace (128 KiB) and the call leaves it zero again
        assert int(got["ws"][:CTL_BYTES].sum()) == 0


def test_decode_edge_lengths_dense_equivalence():
    """Every length around the 512-block boundary, 1..4 verify queries."""
    need_gpu()
    lens, nq = [], []
    for L in list(range(1, 13)) + list(range(2044, 2060)) + [4099, 8195]:
        for n in (1, 4):
            if n <= L:
                lens.append(L)
                nq.append(n)
    w = make_custom("edges", lens, nq, 16, 2, seed=701)
    say("qsa_decode edges", len(lens), "requests")
    ref = oracle_decode(w, want_scores=False)
    got = run_decode(w)
    assert_selection_equal(got, ref)
    assert_out_close(got["out"], ref["out"])
    assert_lean_decode_same(w, got)
    # length 1: the output is the single V row itself
    for r in range(w.num_req):
        if int(w.seq_len[r]) == 1:
            qi = int(w.q_start[r])
            v = oracle.bf16_to_f64(w.v_cache[int(w.kv_start[r])])
            np.testing.assert_allclose(got["out"][qi], np.repeat(v, 8, axis=0), rtol=1e-6, atol=1e-6)


def test_decode_no_full_blocks():
    """Batches where no request has a full 4-token block (max_blocks = 0: no
    scoring launch, nothing to select): every query attends over its partial
    block only, as dense attention over its 1-3 tokens; also a single token."""
    need_gpu()
    for lens, nq, kv in (([1, 2, 3, 3, 2], [1, 2, 3, 1, 2], "bf16"), ([3, 1], [3, 1], "fp8_e4m3"), ([1], [1], "bf16")):
        w = make_custom("nofull", lens, nq, 8, 2, kv_dtype=kv, seed=811 + len(lens))
        say("qsa_decode without full blocks", lens, nq, kv)
        assert batch_of(w).max_blocks == 0
        ref = oracle_decode(w, want_scores=False)
        got = run_decode(w)
        assert_selection_equal(got, ref)
        assert np.all(got["n_pos"] == np.array([int(x) for x in ref["n_pos"]]))
        assert_out_close(got["out"], ref["out"])
        assert_lean_decode_same(w, got)


def test_decode_small_k():
    need_gpu()
    w = _mixed_workload(seed=801)
    for k in (1, 16, 100):
        say("qsa_decode k", k)
        ref = oracle_decode(w, want_scores=False, k=k)
        got = run_decode(w, k=k)
        assert_selection_equal(got, ref)
        assert_out_close(got["out"], ref["out"])
        assert_lean_decode_same(w, got, k=k)


def test_decode_deterministic_and_workspace_reusable():
    need_gpu()
    w = _mixed_workload(kv="fp8_e4m3", seed=901)
    say("qsa_decode determinism", w.name)
    dev = upload(w)
    a = run_decode(w, dev)
    # one workspace serves consecutive calls (each call leaves it reusable)
    b = run_decode(w, dev, ws=a["ws"])
    c = run_decode(w, dev, ws=a["ws"])
    for x in (b, c):
        assert np.array_equal(a["out"].view(np.uint64), x["out"].view(np.uint64))
        assert np.array_equal(a["pos"], x["pos"])
    # the production call on the same workspace, twice, then the checked call again
    for _ in range(2):
        lean = run_decode(w, dev, ws=a["ws"], debug=False)
        assert np.array_equal(a["out"].view(np.uint64), lean["out"].view(np.uint64))
    d = run_decode(w, dev, ws=a["ws"])
    assert np.array_equal(a["out"].view(np.uint64), d["out"].view(np.uint64))
    assert np.array_equal(a["pos"], d["pos"])

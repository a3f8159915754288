"""GPU parity of the rows past the core path: compressed-key append, paged KV
caches, and selection reuse by later MTP draft steps.  Every case compares the
HIP path with the oracle on the same seeded bytes: keys, selections and
positions bit for bit, outputs within 2e-3 * max|out|."""
import numpy as np
import pytest
import torch

import block_sparse_attention_qsa_amd as qsa
import oracle
from workloads import bf16_bits_from_f32, make_custom
from workloads.device import upload
from gpu_helpers import (SM_SCALE, assert_out_close, assert_selection_equal, bf16_dev, decode_paged, need_gpu,
                         run_decode, say)

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _token_keys(rng, n):
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x[rng.random((n, 128)) < 0.05] = 0.0
    x[:, :4] *= np.float32(1e-38)                       # subnormal BF16 range
    x[:, 4:8] = rng.integers(-8, 9, (n, 4)).astype(np.float32)
    return bf16_bits_from_f32(x)


@pytest.mark.parametrize("paged", [False, True])
def test_compress_keys(paged):
    need_gpu()
    rng = np.random.default_rng(700 + paged)
    seq = rng.integers(1, 3000, 24)
    seq[0], seq[1], seq[2] = 4, 7, 2001                  # a block at the start, nothing, a prefill
    step = rng.integers(0, 9, 24)
    prev = np.maximum(seq - step, 0)
    prev[2] = 0
    nreq = len(seq)
    rows = seq // 4
    blk_start = np.concatenate([[0], np.cumsum(rows + 3)[:-1]])   # gaps between requests' key rows
    kv_start = np.concatenate([[5], 5 + np.cumsum(seq + 11)[:-1]])
    slots = int(kv_start[-1] + seq[-1] + 64)
    page_size, table = 16, None
    if paged:
        pages = -(-seq // page_size)
        table = np.zeros((nreq, int(pages.max())), np.int64)
        perm = rng.permutation(int(pages.sum()) + 5)
        table_flat = perm[:int(pages.sum())]
        off = 0
        for r in range(nreq):
            table[r, :pages[r]] = table_flat[off:off + pages[r]]
            off += pages[r]
        slots = int((table.max() + 1) * page_size)
    tok = _token_keys(rng, slots)
    nrows = int(blk_start[-1] + rows[-1] + 8)
    ck_init = np.full((nrows, 128), 0x7E7E, np.uint16)
    ck = bf16_dev(ck_init)
    b = qsa.Batch(np.arange(nreq + 1), seq, None if paged else kv_start, blk_start,
                  page_table=table, page_size=page_size if paged else None)
    say("qsa_compress_keys paged" if paged else "qsa_compress_keys", nreq, "requests")
    qsa.qsa_compress_keys(b, torch.from_numpy(prev.astype(np.int32)).cuda(), bf16_dev(tok), ck)
    torch.cuda.synchronize()
    got = _bits(ck)
    want = ck_init.copy()
    for r in range(nreq):
        keys = oracle.compress_new_keys(int(seq[r]), int(prev[r]), tok, int(kv_start[r]),
                                        None if table is None else table[r], page_size if paged else None)
        for bi, key in keys.items():
            want[blk_start[r] + bi] = key
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kv,page_size", [("bf16", 16), ("fp8_e4m3", 64), ("bf16", 4)])
def test_paged_decode(kv, page_size):
    need_gpu()
    w = make_custom("paged", [9000, 3001, 57, 20003, 2052], [4, 2, 1, 4, 3], 32, 4, kv_dtype=kv, seed=710)
    say("paged qsa_decode", kv, "page size", page_size)
    got, table, kc, vc = decode_paged(w, page_size, 711)
    ref = oracle.decode(w.q_start, w.seq_len, w.kv_start, w.blk_start, w.idx_q, w.ckeys, w.q, kc, vc,
                        w.kv_dtype, w.k_scale, w.v_scale, sm_scale=SM_SCALE, want_scores=False,
                        page_table=table, page_size=page_size)
    assert_selection_equal(got, ref)
    assert_out_close(got["out"], ref["out"])
    # the same logical cache, contiguous: identical selection and identical output bits
    flat = run_decode(w)
    assert np.array_equal(flat["sel"], got["sel"])
    assert np.array_equal(flat["out"].view(np.uint64), got["out"].view(np.uint64))


def test_paged_decode_long_row():
    """Paged KV with a row past 32,768 blocks (140,000 tokens): the two-step
    long-row selection writes positions through the page table."""
    need_gpu()
    w = make_custom("paged-long", [140000, 57, 3001], [4, 1, 2], 16, 2, kv_dtype="fp8_e4m3", seed=712)
    say("paged qsa_decode, long row")
    got, table, kc, vc = decode_paged(w, 64, 713)
    ref = oracle.decode(w.q_start, w.seq_len, w.kv_start, w.blk_start, w.idx_q, w.ckeys, w.q, kc, vc,
                        w.kv_dtype, w.k_scale, w.v_scale, sm_scale=SM_SCALE, want_scores=False,
                        page_table=table, page_size=64)
    assert_selection_equal(got, ref)
    assert_out_close(got["out"], ref["out"])


def test_draft_steps_reuse_selection():
    """A verify step selects; later draft steps of each request (after 1..4
    accepted tokens, then 0..2 more drafted ones) reuse the selection of the
    request's last verify query through qsa_build_index - blocks that are not
    full at the draft's length are dropped - and attend with qsa_sparse_attn."""
    need_gpu()
    w = make_custom("draft", [12345, 50000, 2100, 777], [4, 4, 3, 2], 32, 4, kv_dtype="bf16", seed=720)
    dev = upload(w)
    say("verify step")
    ver = run_decode(w, dev)
    rng = np.random.default_rng(721)
    k = qsa.TOPK
    for d in range(3):
        acc = [int(rng.integers(1, int(w.q_start[r + 1] - w.q_start[r]) + 1)) for r in range(w.num_req)]
        # one draft query per request, causal length = accepted prefix + d drafted tokens
        seq = [int(w.seq_len[r]) - int(w.q_start[r + 1] - w.q_start[r]) + acc[r] + d for r in range(w.num_req)]
        src = [int(w.q_start[r]) + acc[r] - 1 for r in range(w.num_req)]        # query vectors
        last = [int(w.q_start[r + 1]) - 1 for r in range(w.num_req)]            # reused selections
        sel = torch.from_numpy(ver["sel"][last].copy()).cuda()
        n_sel = torch.from_numpy(ver["n_sel"][last].copy()).cuda()
        b = qsa.Batch(np.arange(w.num_req + 1), seq, w.kv_start, w.blk_start)
        pos = torch.full((w.num_req, 4 * k + 3), -7, dtype=torch.int32, device="cuda")
        n_pos = torch.full((w.num_req,), -7, dtype=torch.int32, device="cuda")
        qsa.qsa_build_index(b, sel, n_sel, pos, n_pos)
        qd = torch.from_numpy(w.q[src].copy().view(np.int16)).cuda().view(torch.bfloat16)
        out = torch.full((w.num_req, w.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
        ws = qsa.alloc_workspace(b, w.num_q_heads, w.num_kv_heads, k)
        say("draft step", d, "accepted", acc)
        qsa.qsa_sparse_attn(b, qd, dev["k_cache"], dev["v_cache"], pos, n_pos, out, sm_scale=SM_SCALE, workspace=ws)
        torch.cuda.synchronize()
        ref_out = np.zeros((w.num_req, w.num_q_heads, 128))
        for r in range(w.num_req):
            rp, rn = oracle.build_positions(ver["sel"][last[r], :ver["n_sel"][last[r]]], seq[r], int(w.kv_start[r]), k)
            assert n_pos[r].item() == rn and np.array_equal(pos[r].cpu().numpy(), rp)
            rows = rp[:rn]
            kr, vr = oracle.bf16_to_f64(w.k_cache[rows]), oracle.bf16_to_f64(w.v_cache[rows])
            ref_out[r] = oracle.sparse_attention(oracle.bf16_to_f64(w.q[src[r]]), kr, vr, SM_SCALE)
        assert_out_close(out.cpu().numpy().astype(np.float64), ref_out)

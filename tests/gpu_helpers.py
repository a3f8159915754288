"""Shared helpers of the GPU parity tests: upload a workload, run the oracle on
the same bytes, compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_qsa_amd as qsa
import oracle
from workloads import paged_layout
from workloads.device import upload

SM_SCALE = 1.0 / math.sqrt(128)
OUT_TOL = 2e-3          # max |gpu - oracle| <= OUT_TOL * max |oracle|


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    qsa.lib()   # raises if the HIP library is not built


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def batch_of(w) -> qsa.Batch:
    return qsa.Batch(w.q_start, w.seq_len, w.kv_start, w.blk_start)


def oracle_decode(w, **kw):
    return oracle.decode(w.q_start, w.seq_len, w.kv_start, w.blk_start, w.idx_q, w.ckeys, w.q,
                         w.k_cache, w.v_cache, w.kv_dtype, w.k_scale, w.v_scale, sm_scale=SM_SCALE, **kw)


def run_decode(w, dev=None, out_dtype=torch.float32, k=qsa.TOPK, ws=None, debug=True):
    """Fused qsa_decode.  debug=True also asks for sel / n_sel / pos; without
    them (the production call) only out and n_pos come back."""
    dev = upload(w) if dev is None else dev
    b = batch_of(w)
    hq = w.num_q_heads
    width = 4 * k + 3
    out = torch.full((w.num_q, hq, 128), float("nan"), dtype=out_dtype, device="cuda")
    n_pos = torch.full((w.num_q,), -7, dtype=torch.int32, device="cuda")
    ws = qsa.alloc_workspace(b, hq, w.num_kv_heads, k) if ws is None else ws
    extra = {}
    if debug:
        extra = {"sel": torch.full((w.num_q, k), -7, dtype=torch.int32, device="cuda"),
                 "n_sel": torch.full((w.num_q,), -7, dtype=torch.int32, device="cuda"),
                 "pos": torch.full((w.num_q, width), -7, dtype=torch.int32, device="cuda")}
    qsa.qsa_decode(b, dev["idx_q"], dev["ckeys"], dev["q"], dev["k_cache"], dev["v_cache"], out, ws,
                   k_scale=dev["k_scale"], v_scale=dev["v_scale"], k=k, sm_scale=SM_SCALE, n_pos=n_pos, **extra)
    torch.cuda.synchronize()
    res = {"out": out.float().cpu().numpy().astype(np.float64), "n_pos": n_pos.cpu().numpy(), "ws": ws}
    for key, t in extra.items():
        res[key] = t.cpu().numpy()
    return res


def assert_lean_decode_same(w, got, dev=None, k=qsa.TOPK, out_dtype=torch.float32):
    """The production call (no sel / n_sel / pos requested, as a serving loop
    makes it) gives the same n_pos and the same output bits as the checked
    call."""
    lean = run_decode(w, dev, out_dtype=out_dtype, k=k, debug=False)
    assert np.array_equal(lean["n_pos"], got["n_pos"])
    assert np.array_equal(lean["out"].view(np.uint64), got["out"].view(np.uint64))
    return lean


def assert_selection_equal(got, ref, queries=None):
    qs = range(ref["sel"].shape[0]) if queries is None else queries
    for qi in qs:
        assert got["n_sel"][qi] == ref["n_sel"][qi], (qi, got["n_sel"][qi], ref["n_sel"][qi])
        assert np.array_equal(got["sel"][qi], ref["sel"][qi]), qi
        assert got["n_pos"][qi] == ref["n_pos"][qi], qi
        assert np.array_equal(got["pos"][qi], ref["pos"][qi]), qi


def out_errors(gpu_out, ref_out, queries=None):
    qs = np.arange(ref_out.shape[0]) if queries is None else np.asarray(queries)
    g, r = gpu_out[qs], ref_out[qs]
    assert np.all(np.isfinite(g))
    cfg = float(np.abs(g - r).max() / np.abs(r).max())
    per_q = float(max(np.abs(g[i] - r[i]).max() / np.abs(r[i]).max() for i in range(len(qs))))
    return cfg, per_q


def assert_out_close(gpu_out, ref_out, queries=None, tol=OUT_TOL):
    cfg, per_q = out_errors(gpu_out, ref_out, queries)
    say(f"out error: config {cfg:.3e}, worst query {per_q:.3e} (bar {tol})")
    assert cfg <= tol, cfg
    assert per_q <= tol, per_q
    return cfg, per_q


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def decode_paged(w, page_size, seed, dev=None, k=qsa.TOPK):
    """qsa_decode of workload w through a paged copy of its KV cache (pages of
    page_size tokens scattered by a seeded permutation); also checks that the
    production call and the stage path (qsa_build_index on the selection)
    agree with it bit for bit.  Returns (results, page table, K, V pages)."""
    table, kc, vc = paged_layout(w, page_size, seed)
    d = upload(w) if dev is None else dict(dev)
    if w.kv_dtype == "bf16":
        d["k_cache"], d["v_cache"] = bf16_dev(kc), bf16_dev(vc)
    else:
        d["k_cache"] = torch.from_numpy(np.ascontiguousarray(kc)).cuda().view(torch.float8_e4m3fn)
        d["v_cache"] = torch.from_numpy(np.ascontiguousarray(vc)).cuda().view(torch.float8_e4m3fn)
    b = qsa.Batch(w.q_start, w.seq_len, None, w.blk_start, page_table=table, page_size=page_size)
    hq = w.num_q_heads
    out = torch.full((w.num_q, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((w.num_q, k), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((w.num_q,), -7, dtype=torch.int32, device="cuda")
    pos = torch.full((w.num_q, 4 * k + 3), -7, dtype=torch.int32, device="cuda")
    n_pos = torch.full((w.num_q,), -7, dtype=torch.int32, device="cuda")
    ws = qsa.alloc_workspace(b, hq, w.num_kv_heads, k)
    qsa.qsa_decode(b, d["idx_q"], d["ckeys"], d["q"], d["k_cache"], d["v_cache"], out, ws, k_scale=d["k_scale"],
                   v_scale=d["v_scale"], k=k, sm_scale=SM_SCALE, sel=sel, n_sel=n_sel, pos=pos, n_pos=n_pos)
    # the production call (no sel / n_sel / pos requested)
    out_lean = torch.full_like(out, float("nan"))
    n_pos_lean = torch.full_like(n_pos, -7)
    qsa.qsa_decode(b, d["idx_q"], d["ckeys"], d["q"], d["k_cache"], d["v_cache"], out_lean, ws,
                   k_scale=d["k_scale"], v_scale=d["v_scale"], k=k, sm_scale=SM_SCALE, n_pos=n_pos_lean)
    # the stage path: selection without positions, then the index builder
    pos2 = torch.full_like(pos, -7)
    n_pos2 = torch.full_like(n_pos, -7)
    qsa.qsa_build_index(b, sel, n_sel, pos2, n_pos2, k=k)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy().astype(np.float64), "sel": sel.cpu().numpy(), "n_sel": n_sel.cpu().numpy(),
           "pos": pos.cpu().numpy(), "n_pos": n_pos.cpu().numpy()}
    assert np.array_equal(pos2.cpu().numpy(), res["pos"]) and np.array_equal(n_pos2.cpu().numpy(), res["n_pos"])
    assert np.array_equal(n_pos_lean.cpu().numpy(), res["n_pos"])
    assert np.array_equal(out_lean.cpu().numpy().view(np.uint32), out.cpu().numpy().view(np.uint32))
    return res, table, kc, vc

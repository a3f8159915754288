"""qsa_decode captured in a HIP graph, the form a serving loop (and the
benchmark) runs it in: several calls on two input sets in one graph, replayed
several times with eager work and synchronisations between the replays.

Every replay must reproduce the eager calls' outputs and n_pos bit for bit and
leave the workspace's control region zero; the eager outputs of the first
input set are checked against the oracle.  Three batches take the three
launch forms of the step: a uniform 4-query batch (split attention with the
in-kernel merge), a ragged batch (the attention's work list, written by the
selection launch) and a row past 32,768 blocks (two-step selection).  The
allocation-free entry point is captured the same way."""
import numpy as np
import pytest
import torch

import block_sparse_attention_qsa_amd as qsa
from workloads import make_custom
from workloads.device import upload
from gpu_helpers import SM_SCALE, assert_out_close, batch_of, need_gpu, oracle_decode, say

pytestmark = pytest.mark.gpu

CTL_BYTES = 128 * 1024
CALLS = 4          # calls per graph: call i reads input set i % 2 and writes output i
REPLAYS = 3

CASES = {
    # name: (lengths, queries per request, Hq, Hkv, KV dtype)
    "uniform": ([50_000], [4], 32, 4, "bf16"),
    "ragged": ([37, 3_000, 20_000, 9_001, 130, 2_051], [1, 4, 4, 2, 1, 3], 32, 4, "fp8_e4m3"),
    "long_row": ([140_000], [4], 16, 2, "bf16"),
}


def _inputs(name, seed):
    lens, nq, hq, hkv, kv = CASES[name]
    # no layout gaps: both input sets share one batch layout
    return make_custom(f"graph_{name}_{seed}", lens, nq, hq, hkv, kv_dtype=kv, seed=seed, index_values="normal",
                       gaps=False)


def _call(fn, b, dev, out, n_pos, **kw):
    fn(b, dev["idx_q"], dev["ckeys"], dev["q"], dev["k_cache"], dev["v_cache"], out, k_scale=dev["k_scale"],
       v_scale=dev["v_scale"], sm_scale=SM_SCALE, n_pos=n_pos, **kw)


def _run_graph_case(name, static):
    need_gpu()
    ws_ = [_inputs(name, 7100 + s) for s in range(2)]
    b = batch_of(ws_[0])
    w0 = ws_[0]
    devs = [upload(w) for w in ws_]
    nq, hq = w0.num_q, w0.num_q_heads
    outs = [torch.empty((nq, hq, 128), dtype=torch.float32, device="cuda") for _ in range(CALLS)]
    npos = [torch.empty((nq,), dtype=torch.int32, device="cuda") for _ in range(CALLS)]
    if static:
        ws = None
        fn = qsa.qsa_decode_static
    else:
        ws = qsa.alloc_workspace(b, hq, w0.num_kv_heads)

        def fn(b_, *a, **kw):   # a: idx_q, ckeys, q, k_cache, v_cache, out
            qsa.qsa_decode(b_, *a, ws, **kw)

    def step(i):
        _call(fn, b, devs[i % 2], outs[i], npos[i])

    # eager reference calls (these also make the static scratch's first-call set-up happen outside the graph)
    for o, p in zip(outs, npos):
        o.fill_(float("nan"))
        p.fill_(-7)
    for i in range(CALLS):
        step(i)
    torch.cuda.synchronize()
    eager = [(o.cpu().numpy().copy(), p.cpu().numpy().copy()) for o, p in zip(outs, npos)]
    for i in range(2, CALLS):
        assert np.array_equal(eager[i][0].view(np.uint32), eager[i % 2][0].view(np.uint32)), i
    say(name, "oracle")
    ref = oracle_decode(w0, want_scores=False)
    assert np.array_equal(eager[0][1], ref["n_pos"])
    assert_out_close(eager[0][0].astype(np.float64), ref["out"])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(CALLS):
            step(i)
    torch.cuda.synchronize()
    a = torch.randn(512, 512, device="cuda")
    for rep in range(REPLAYS):
        say(name, "static" if static else "workspace", "replay", rep)
        for o, p in zip(outs, npos):
            o.fill_(float("nan"))
            p.fill_(-7)
        a = torch.tanh(a @ a.t() * 1e-3)       # eager work of the program between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, p) in enumerate(zip(outs, npos)):
            assert np.array_equal(p.cpu().numpy(), eager[i][1]), (rep, i)
            assert np.array_equal(o.cpu().numpy().view(np.uint32), eager[i][0].view(np.uint32)), (rep, i)
        if ws is not None:
            assert int(ws[:CTL_BYTES].sum().item()) == 0
    del g
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", list(CASES))
def test_decode_graph_replays_match_eager(name):
    _run_graph_case(name, static=False)


@pytest.mark.parametrize("name", ["uniform", "ragged"])
def test_static_decode_graph_replays_match_eager(name):
    _run_graph_case(name, static=True)

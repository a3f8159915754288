"""Fused qsa_decode against the oracle on seeded random small batches.

Each case draws its batch size, verify-query counts, context lengths (tiny
ones with only a partial block, ones around the 512-block selection boundary,
and long ones past 16,384 blocks), KV head count, GQA group size, KV dtype,
output dtype, k and index-value style, so that combinations no hand-written
case names are still checked: selection and positions bit for bit, the output
within the FP32 bar (BF16 output: one extra rounding on top), and the
production call (no debug outputs) to the bit against the checked call.
"""
import numpy as np
import pytest
import torch

from workloads import make_custom
from workloads.device import upload
from gpu_helpers import (OUT_TOL, SM_SCALE, assert_lean_decode_same, assert_out_close, assert_selection_equal,
                         decode_paged, need_gpu, oracle_decode, run_decode, say)

pytestmark = pytest.mark.gpu

MAX_TOTAL_TOKENS = 200_000   # keeps the host-side KV caches of a case small


def _case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    lens = []
    for _ in range(B):
        kind = int(rng.integers(0, 4))
        if kind == 0:
            L = int(rng.integers(1, 64))          # a few blocks, often only a partial one
        elif kind == 1:
            L = int(rng.integers(2040, 2060))     # around 512 full blocks
        elif kind == 2:
            L = int(rng.integers(2060, 20000))
        else:
            L = int(rng.integers(65540, 70000))   # past 16,384 blocks
        lens.append(L)
    while sum(lens) > MAX_TOTAL_TOKENS:
        i = int(np.argmax(lens))
        lens[i] //= 2
    nq = [int(rng.integers(1, min(4, L) + 1)) for L in lens]
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8, 16] if hkv <= 4 else [1, 2, 4]))
    kv = str(rng.choice(["bf16", "fp8_e4m3"]))
    k = int(rng.choice([512, 512, 100, 1]))
    out_bf16 = bool(rng.integers(0, 4) == 0)
    iv = str(rng.choice(["int", "normal"]))
    return lens, nq, hkv, group, kv, k, out_bf16, iv


@pytest.mark.parametrize("seed", list(range(64)))
def test_random_decode(seed):
    need_gpu()
    lens, nq, hkv, group, kv, k, out_bf16, iv = _case(1000 + seed)
    say(f"case {seed}: lens {lens} nq {nq} Hkv {hkv} G {group} {kv} k {k} out {'bf16' if out_bf16 else 'f32'} {iv}")
    w = make_custom(f"rand{seed}", lens, nq, group * hkv, hkv, kv_dtype=kv, seed=2000 + seed, index_values=iv)
    ref = oracle_decode(w, want_scores=False, k=k)
    dev = upload(w)
    out_dtype = torch.bfloat16 if out_bf16 else torch.float32
    got = run_decode(w, dev, k=k, out_dtype=out_dtype)
    assert_selection_equal(got, ref)
    if out_bf16:
        # one BF16 rounding (at most 2^-8 relative) on top of the FP32 bar
        r = ref["out"]
        err = np.abs(got["out"] - r) - 2.0 ** -8 * np.abs(r)
        assert err.max() <= OUT_TOL * np.abs(r).max()
    else:
        assert_out_close(got["out"], ref["out"])
    assert_lean_decode_same(w, got, dev, k=k, out_dtype=out_dtype)


@pytest.mark.parametrize("seed", list(range(32)))
def test_random_decode_paged(seed):
    """The same random batches through a paged KV cache: pages of 4 to 256
    tokens scattered over the cache by a seeded permutation."""
    import oracle
    need_gpu()
    lens, nq, hkv, group, kv, k, _, iv = _case(3000 + seed)
    page_size = int(np.random.default_rng(4000 + seed).choice([4, 8, 16, 64, 256]))
    say(f"paged case {seed}: lens {lens} nq {nq} Hkv {hkv} G {group} {kv} k {k} {iv} page {page_size}")
    w = make_custom(f"randp{seed}", lens, nq, group * hkv, hkv, kv_dtype=kv, seed=5000 + seed, index_values=iv)
    got, table, kc, vc = decode_paged(w, page_size, 6000 + seed, k=k)
    ref = oracle.decode(w.q_start, w.seq_len, w.kv_start, w.blk_start, w.idx_q, w.ckeys, w.q, kc, vc, w.kv_dtype,
                        w.k_scale, w.v_scale, k=k, sm_scale=SM_SCALE, want_scores=False, page_table=table,
                        page_size=page_size)
    assert_selection_equal(got, ref)
    assert_out_close(got["out"], ref["out"])

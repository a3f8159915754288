"""Checks that pin the CPU oracle to facts other than itself.

Each check takes the oracle as an argument (a module or namespace with the
oracle's functions) so that test_oracle_mutations.py can run the same checks
against copies of the oracle with a planted mistake and show they fail.

Sources of truth used here: exact integer / rational arithmetic, brute-force
rank counting, torch's scaled_dot_product_attention and float8 / bfloat16
decoders, closed forms of special cases, and the constants the pages print
(tests/golden/pages_constants.json).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from workloads import make_custom, bf16_bits_from_f32, fp8_e4m3fn_bits_from_f32, paged_layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def pages_constants() -> dict:
    with open(os.path.join(GOLDEN, "pages_constants.json")) as f:
        return json.load(f)


def run_decode(orc, w, **kw):
    return orc.decode(w.q_start, w.seq_len, w.kv_start, w.blk_start, w.idx_q, w.ckeys, w.q,
                      w.k_cache, w.v_cache, w.kv_dtype, w.k_scale, w.v_scale, **kw)


# ---------------------------------------------------------------- decoders
def check_fp8_decode(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.fp8_e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # values fixed by the OCP E4M3 definition
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0        # largest normal
    assert got[0x38] == 1.0 and got[0xB8] == -1.0
    assert got[0x08] == 2.0 ** -6                            # smallest normal
    assert got[0x01] == 2.0 ** -9                            # smallest subnormal
    assert got[0x07] == 7 * 2.0 ** -9                        # largest subnormal
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def check_bf16_decode(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 65536, 4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                  # finite only
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.bf16_to_f64(bits), ref)


# ---------------------------------------------------------------- a1 scores
def check_scores_exact_integer(orc):
    rng = np.random.default_rng(11)
    iq = rng.integers(-8, 9, 128)
    keys = rng.integers(-8, 9, (500, 128))
    s = orc.block_scores(bf16_bits_from_f32(iq.astype(np.float32)),
                         bf16_bits_from_f32(keys.astype(np.float32)))
    exact = keys.astype(np.int64) @ iq.astype(np.int64)      # integer arithmetic
    assert s.dtype == np.float32
    assert np.array_equal(s.astype(np.int64), exact)
    # worst case |s| = 128 * 64 = 8192 is exact in FP32
    s2 = orc.block_scores(bf16_bits_from_f32(np.full(128, -8, np.float32)),
                          bf16_bits_from_f32(np.full((1, 128), 8, np.float32)))
    assert s2[0] == -8192.0


def check_scores_unit_vectors(orc):
    rng = np.random.default_rng(12)
    keys = bf16_bits_from_f32(rng.standard_normal((64, 128)).astype(np.float32))
    for d in (0, 5, 127):
        e = np.zeros(128, np.float32)
        e[d] = 1.0
        s = orc.block_scores(bf16_bits_from_f32(e), keys)
        kd = torch.from_numpy(keys[:, d].astype(np.int16)).view(torch.bfloat16).float().numpy()
        assert np.array_equal(s, kd)


def check_scores_rounded_once(orc):
    """Non-integer BF16 inputs: the FP32 score is the exact rational sum rounded once."""
    rng = np.random.default_rng(13)
    iq = bf16_bits_from_f32(rng.standard_normal(128).astype(np.float32))
    keys = bf16_bits_from_f32(rng.standard_normal((24, 128)).astype(np.float32))
    s = orc.block_scores(iq, keys)
    iqf = torch.from_numpy(iq.astype(np.int16)).view(torch.bfloat16).double().numpy()
    kf = torch.from_numpy(keys.astype(np.int16)).view(torch.bfloat16).double().numpy()
    for b in range(keys.shape[0]):
        exact = sum(Fraction(float(a)) * Fraction(float(c)) for a, c in zip(iqf, kf[b]))
        assert s[b] == _nearest_f32(exact)


def _nearest_f32(fr: Fraction) -> np.float32:
    x = np.float32(float(fr))
    cands = [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1))


# ---------------------------------------------------------------- a2 selection
def _brute_force_select(scores, k):
    s = [float(x) for x in scores]
    n = len(s)
    keep = []
    for b in range(n):
        rank = sum(1 for c in range(n) if s[c] > s[b]) + sum(1 for c in range(b) if s[c] == s[b])
        if rank < k:
            keep.append(b)
    return np.array(keep, dtype=np.int64)


def check_select_bruteforce(orc):
    rng = np.random.default_rng(21)
    for trial in range(40):
        n = int(rng.integers(1, 260))
        k = int(rng.integers(1, 40))
        levels = int(rng.integers(1, 12))                    # few distinct values -> many ties
        scores = rng.integers(-levels, levels + 1, n).astype(np.float32) * np.float32(0.5)
        if trial % 4 == 0:
            scores = rng.standard_normal(n).astype(np.float32)
        got = orc.select_blocks(scores, k)
        assert np.array_equal(got, _brute_force_select(scores, k)), (trial, n, k)


def check_select_threshold_straddle(orc):
    """300 blocks at score A, 400 at B < A, the rest lower: keep all A and the
    212 lowest-index B blocks."""
    rng = np.random.default_rng(22)
    n = 2000
    perm = rng.permutation(n)
    scores = np.full(n, -5.0, np.float32)
    a_idx, b_idx = perm[:300], perm[300:700]
    scores[a_idx] = 9.0
    scores[b_idx] = 3.0
    scores[perm[700:]] = rng.uniform(-100, 2.9, n - 700).astype(np.float32)
    want = np.sort(np.concatenate([a_idx, np.sort(b_idx)[:212]]))
    assert np.array_equal(orc.select_blocks(scores, 512), want)


def check_select_all_when_few(orc):
    for nf in (0, 1, 7, 511, 512):
        s = np.random.default_rng(nf).standard_normal(nf).astype(np.float32)
        assert np.array_equal(orc.select_blocks(s, 512), np.arange(nf))


def check_select_signed_zero(orc):
    scores = np.array([-0.0, 0.0, -1.0, 0.0, -0.0, 2.0], np.float32)
    # ranks: 2.0 first, then the four zeros in index order, then -1
    assert np.array_equal(orc.select_blocks(scores, 3), np.array([0, 1, 5]))
    assert np.array_equal(orc.select_blocks(scores, 5), np.array([0, 1, 3, 4, 5]))


def check_select_tie_construction(orc):
    """~5% of blocks share the strict maximum; each query keeps the k lowest
    indices of that tie set among its own full blocks (closed form)."""
    w = make_custom("ties", [16384, 16387], [4, 3], 8, 1, seed=5, tie_fraction=0.05)
    k = 64
    res = run_decode(orc, w, k=k)
    for r in range(w.num_req):
        tie = w.meta["tie_sets"][r]
        nq = int(w.q_start[r + 1] - w.q_start[r])
        for j in range(nq):
            qi = int(w.q_start[r]) + j
            nf = (int(w.seq_len[r]) - nq + 1 + j) // 4
            want = np.sort(tie[tie < nf])[:k]
            assert np.array_equal(res["sel"][qi, :k], want), (r, j)


# ---------------------------------------------------------------- a3 positions
def check_positions_invariants(orc):
    k = 512
    const = pages_constants()
    width = 4 * k + 3
    assert orc.WIDTH == const["selection_buffer_width"] == width
    assert orc.BLOCK == const["block_tokens"] and orc.TOPK == const["max_full_blocks_per_query"]
    rng = np.random.default_rng(31)
    for L in [1, 2, 3, 4, 5, 8, 2047, 2048, 2049, 2050, 2051, 2052, 2055, 3000, 50000]:
        nf = L // 4
        s = rng.integers(-20, 20, nf).astype(np.float32)
        sel = orc.select_blocks(s, k)
        kv0 = int(rng.integers(0, 100))
        pos, n = orc.build_positions(sel, L, kv0, k)
        assert pos.shape == (width,)
        assert n == 4 * min(nf, k) + L % 4
        v = pos[:n]
        assert np.all(pos[n:] == -1)
        assert np.all(np.diff(v) > 0)                        # strictly ascending
        assert v.min() >= kv0 and v.max() < kv0 + L
        for b in sel:                                        # every kept block, all 4 slots
            assert np.all(np.isin(kv0 + 4 * b + np.arange(4), v))
        assert np.all(np.isin(np.arange(kv0 + 4 * nf, kv0 + L), v))   # partial block kept
        assert n <= const["selection_buffer_width"]
        assert 4 * min(nf, k) <= const["max_selected_positions"]


def check_positions_mtp_lengths(orc):
    """50,000-token request with 4 verify queries: causal prefixes 49,997..50,000,
    so the kept partial blocks hold 1, 2, 3, 0 tokens and n_pos is
    2,049 / 2,050 / 2,051 / 2,048."""
    w = make_custom("mtp", [50000], [4], 8, 1, seed=3)
    res = run_decode(orc, w, want_scores=False)
    assert list(res["n_pos"]) == [2049, 2050, 2051, 2048]
    assert list(res["n_sel"]) == [512] * 4
    # queries 0..2 keep their partial block, so their last position is their own
    # newest token, slot kv_start + 49,996 + j; query 3 has no partial block
    for j in range(3):
        assert res["pos"][j, res["n_pos"][j] - 1] == w.kv_start[0] + 49996 + j
    assert res["pos"][3, 2047] < w.kv_start[0] + 50000
    # a single decode query over 8,192 tokens: 2,048 positions, no partial block
    w1 = make_custom("one", [8192], [1], 8, 1, seed=4)
    r1 = run_decode(orc, w1, want_scores=False)
    assert r1["n_pos"][0] == 2048


# ---------------------------------------------------------------- a4 attention
def _dense_sdpa(w, r, j, sm_scale):
    """Textbook attention of verify query j of request r over its whole causal
    prefix, by torch SDPA in float64 (GQA by repeat_interleave of KV heads)."""
    nq = int(w.q_start[r + 1] - w.q_start[r])
    L = int(w.seq_len[r]) - nq + 1 + j
    qi = int(w.q_start[r]) + j
    sl = slice(int(w.kv_start[r]), int(w.kv_start[r]) + L)
    return _sdpa_rows(w, qi, np.arange(sl.start, sl.stop), sm_scale)


def _deq_torch(cache, rows, kv_dtype, scale):
    t = torch.from_numpy(np.ascontiguousarray(cache[rows]))
    if kv_dtype == "bf16":
        return t.view(torch.int16).view(torch.bfloat16).double()
    x = t.view(torch.float8_e4m3fn).double()
    return x * torch.from_numpy(scale.astype(np.float64))[None, :, None]


def _sdpa_rows(w, qi, rows, sm_scale):
    G = w.num_q_heads // w.num_kv_heads
    qt = torch.from_numpy(w.q[qi].astype(np.int16)).view(torch.bfloat16).double()   # [Hq, d]
    kt = _deq_torch(w.k_cache, rows, w.kv_dtype, w.k_scale)                         # [n, Hkv, d]
    vt = _deq_torch(w.v_cache, rows, w.kv_dtype, w.v_scale)
    kt = kt.permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()              # [Hq, n, d]
    vt = vt.permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt[:, None, :], kt, vt, scale=sm_scale)
    return o[:, 0, :].numpy()


def check_attention_dense_equivalence(orc):
    """With at most 512 full blocks everything is kept, so the output equals
    dense causal attention over the query's whole prefix."""
    lens = [1, 2, 3, 4, 5, 9, 700, 2047, 2048, 2049, 2050, 2051, 2052, 2054]
    nq = [1, 2, 3, 4, 4, 4, 1, 4, 4, 4, 4, 4, 4, 4]
    for kv in ("bf16", "fp8_e4m3"):
        w = make_custom("dense", lens, nq, 8, 2, kv_dtype=kv, seed=41)
        sm = 1.0 / math.sqrt(128)
        res = run_decode(orc, w, want_scores=False, sm_scale=sm)
        for r in range(w.num_req):
            for j in range(int(w.q_start[r + 1] - w.q_start[r])):
                qi = int(w.q_start[r]) + j
                L = int(w.seq_len[r]) - (int(w.q_start[r + 1] - w.q_start[r])) + 1 + j
                if L // 4 > 512:
                    continue
                ref = _dense_sdpa(w, r, j, sm)
                np.testing.assert_allclose(res["out"][qi], ref, rtol=1e-11, atol=1e-12)


def check_attention_over_selection(orc):
    """Beyond 512 blocks the output equals SDPA over exactly the gathered rows.
    K and V scales are made unequal so that swapping them is visible."""
    w = make_custom("sparse", [9000, 12345], [4, 2], 16, 2, kv_dtype="fp8_e4m3", seed=42)
    w.k_scale = (w.k_scale * np.float32(0.5)).astype(np.float32)
    w.v_scale = (w.v_scale * np.float32(1.75)).astype(np.float32)
    sm = 1.0 / math.sqrt(128)
    res = run_decode(orc, w, want_scores=False, sm_scale=sm)
    for qi in range(w.num_q):
        rows = res["pos"][qi, :res["n_pos"][qi]].astype(np.int64)
        np.testing.assert_allclose(res["out"][qi], _sdpa_rows(w, qi, rows, sm), rtol=1e-11, atol=1e-12)


def check_attention_special_cases(orc):
    rng = np.random.default_rng(51)
    d = 128
    # one row: output is that row's V, exactly
    qh = rng.standard_normal((8, d))
    kr = rng.standard_normal((1, 2, d))
    vr = rng.standard_normal((1, 2, d))
    o = orc.sparse_attention(qh, kr, vr, 0.1)
    assert np.array_equal(o[:4], np.repeat(vr[:, 0, :], 4, axis=0))
    assert np.array_equal(o[4:], np.repeat(vr[:, 1, :], 4, axis=0))
    # K == 0: uniform weights, output is the mean of V rows of the head's group
    n = 37
    kr = np.zeros((n, 2, d))
    vr = rng.standard_normal((n, 2, d))
    o = orc.sparse_attention(qh, kr, vr, 0.1)
    np.testing.assert_allclose(o[0], vr[:, 0, :].mean(0), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[7], vr[:, 1, :].mean(0), rtol=1e-13, atol=1e-14)
    # constant V: output is that constant
    kr = rng.standard_normal((n, 2, d))
    vr = np.full((n, 2, d), 0.375)
    np.testing.assert_allclose(orc.sparse_attention(qh, kr, vr, 0.09), 0.375, rtol=1e-14)
    # convex combination: every component inside [min, max] of its V column
    vr = rng.standard_normal((n, 2, d))
    o = orc.sparse_attention(qh, kr, vr, 0.09)
    for h in range(8):
        g = h // 4
        assert np.all(o[h] <= vr[:, g, :].max(0) + 1e-12) and np.all(o[h] >= vr[:, g, :].min(0) - 1e-12)
    # permutation of the gathered rows does not change the output
    perm = rng.permutation(n)
    np.testing.assert_allclose(orc.sparse_attention(qh, kr[perm], vr[perm], 0.09), o, rtol=1e-12, atol=1e-14)
    # a large scale concentrates all weight on the best row
    qh1 = np.zeros((8, d)); qh1[:, 0] = 1.0
    kr1 = np.zeros((n, 2, d)); kr1[:, :, 0] = np.arange(n)[:, None]
    o = orc.sparse_attention(qh1, kr1, vr, 1e4)
    assert np.array_equal(o[0], vr[n - 1, 0, :])


# ---------------------------------------------------------------- paged KV, reuse
def check_paged_positions(orc):
    """Page-table slots: an identity table reproduces contiguous slots from 0;
    a permuted table maps every logical token t to table[t // P] * P + t % P,
    keeps each block's four slots consecutive, and a paged decode over caches
    re-laid out that way gives bit-identical outputs to the contiguous one."""
    rng = np.random.default_rng(41)
    for P in (4, 16, 64):
        for L in (3, 4, 5, 2051, 2052, 9001):
            nf = L // 4
            sel = orc.select_blocks(rng.integers(-9, 9, nf).astype(np.float32), 512)
            pages = -(-L // P)
            ident = np.arange(pages)
            p_c, n_c = orc.build_positions(sel, L, 0, 512)
            p_i, n_i = orc.build_positions(sel, L, 0, 512, ident, P)
            assert n_i == n_c and np.array_equal(p_i, p_c)
            table = rng.permutation(pages + 7)[:pages]
            p_p, n_p = orc.build_positions(sel, L, 0, 512, table, P)
            assert n_p == n_c
            logical = p_c[:n_c]
            assert np.array_equal(p_p[:n_p], table[logical // P] * P + logical % P)
            runs = p_p[:4 * min(nf, 512)].reshape(-1, 4)
            assert np.all(np.diff(runs, axis=1) == 1)
            assert np.all(p_p[n_p:] == -1)
    w = make_custom("paged", [9000, 3001, 57], [4, 2, 1], 8, 2, seed=42)
    ref = run_decode(orc, w, want_scores=False)
    table, kc, vc = paged_layout(w, 16, 43)
    got = orc.decode(w.q_start, w.seq_len, w.kv_start, w.blk_start, w.idx_q, w.ckeys, w.q, kc, vc,
                     w.kv_dtype, w.k_scale, w.v_scale, want_scores=False, page_table=table, page_size=16)
    assert np.array_equal(got["sel"], ref["sel"]) and np.array_equal(got["n_pos"], ref["n_pos"])
    assert np.array_equal(got["out"], ref["out"])


def check_positions_reuse(orc):
    """A selection reused at a shorter length keeps exactly its blocks below
    the new full-block count, then the new partial block."""
    rng = np.random.default_rng(44)
    L_sel = 20003
    sel = orc.select_blocks(rng.integers(-50, 50, L_sel // 4).astype(np.float32), 512)
    for L in (L_sel, L_sel - 1, L_sel - 3, 16000, 9, 4, 1):
        nf = L // 4
        keep = sel[sel < nf]
        pos, n = orc.build_positions(sel, L, 100, 512)
        assert n == 4 * keep.size + L % 4
        want = np.concatenate([(100 + 4 * keep[:, None] + np.arange(4)).reshape(-1),
                               100 + np.arange(4 * nf, L)])
        assert np.array_equal(pos[:n], want) and np.all(pos[n:] == -1)


def _nearest_bf16_bits(value: Fraction, all_neg_zero: bool) -> int:
    """Brute force: among the BF16 patterns next to float32(value) pick the one
    at the smallest exact distance, ties to the even pattern."""
    if value == 0:
        return 0x8000 if all_neg_zero else 0
    f = np.float32(float(value)).view(np.uint32) >> 16
    best = None
    for cand in range(int(f) - 2, int(f) + 3):
        c = cand & 0xFFFF
        if (c & 0x7F80) == 0x7F80:
            continue
        cv = Fraction(float(np.array([c << 16], np.uint32).view(np.float32)[0]))
        key = (abs(cv - value), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def check_compress_keys(orc):
    """Block keys: the mean of the four token keys rounded once to BF16."""
    bf = lambda x: bf16_bits_from_f32(np.asarray(x, np.float32))
    one, e7, e6 = 1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -6
    cases = [
        ([3, 5, 6, 2], 4.0),                    # exact mean
        ([1, 2, 3, 5], 2.75),                   # exact quarter
        ([one, one, one, e7], None),            # 1 + 2^-9: below half a unit -> 1
        ([one, one, e7, e7], 1.0),              # 1 + 2^-8: tie -> even (1.0)
        ([e6, e6, e7, e7], 1.0 + 2 ** -6),      # 1 + 3*2^-8: tie -> even (1 + 2^-6)
    ]
    for vals, want in cases:
        got = orc.compress_block_key(bf(np.array(vals, np.float32))[:, None].repeat(3, 1))
        if want is not None:
            assert np.all(got == bf(np.float32(want))), (vals, got)
    assert orc.compress_block_key(bf(np.array([one, one, one, e7], np.float32))[:, None])[0] == bf(np.float32(1.0))
    # subnormal BF16 unit is 2^-133: mean of 2^-133 x {1, 1, 1, 0} = 0.75 units -> 1 unit
    tiny = np.array([0x0001, 0x0001, 0x0001, 0x0000], np.uint16)[:, None]
    assert orc.compress_block_key(tiny)[0] == 0x0001
    # signed zeros: -0 only when all four are -0
    z = np.array([0x8000, 0x8000, 0x8000, 0x8000], np.uint16)[:, None]
    assert orc.compress_block_key(z)[0] == 0x8000
    z[2, 0] = 0x0000
    assert orc.compress_block_key(z)[0] == 0x0000
    # brute-force nearest on random normals and wide magnitudes
    rng = np.random.default_rng(45)
    for scale in (1.0, 1e-38, 3e37):
        x = (rng.standard_normal((4, 64)) * scale).astype(np.float32)
        bits = bf(x)
        got = orc.compress_block_key(bits)
        vals = orc.bf16_to_f64(bits)
        for dd in range(64):
            m = sum(Fraction(float(v)) for v in vals[:, dd]) / 4
            assert got[dd] == _nearest_bf16_bits(m, bool(np.all(bits[:, dd] == 0x8000))), (scale, dd)
    # the blocks a step completes: prev_len <= 4b + 3 < seq_len
    tok = bf(rng.standard_normal((40, 8)).astype(np.float32))
    keys = orc.compress_new_keys(23, 6, tok, kv_start=3)
    assert sorted(keys) == [1, 2, 3, 4]
    assert np.array_equal(keys[2], orc.compress_block_key(tok[3 + 8:3 + 12]))
    assert sorted(orc.compress_new_keys(8, 8, tok)) == [] and sorted(orc.compress_new_keys(9, 7, tok)) == [1]


ALL_CHECKS = [
    check_fp8_decode, check_bf16_decode,
    check_scores_exact_integer, check_scores_unit_vectors, check_scores_rounded_once,
    check_select_bruteforce, check_select_threshold_straddle, check_select_all_when_few,
    check_select_signed_zero, check_select_tie_construction,
    check_positions_invariants, check_positions_mtp_lengths,
    check_attention_dense_equivalence, check_attention_over_selection, check_attention_special_cases,
    check_paged_positions, check_positions_reuse, check_compress_keys,
]

"""Plant plausible mistakes in a private copy of the oracle and show that the
pins catch every one of them (CPU only; the real oracle is never modified)."""
import importlib.util
import os

import numpy as np
import pytest

import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "qsa_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant", ORACLE_SRC)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _m_tie_higher_index(m):
    def select_blocks(scores, k=m.TOPK):
        s = np.asarray(scores, np.float32).astype(np.float64)
        nf = s.shape[0]
        if nf <= k:
            return np.arange(nf)
        order = np.lexsort((-np.arange(nf), -s))
        return np.sort(order[:k])
    m.select_blocks = select_blocks


def _m_unsorted_output(m):
    def select_blocks(scores, k=m.TOPK):
        s = np.asarray(scores, np.float32).astype(np.float64)
        nf = s.shape[0]
        if nf <= k:
            return np.arange(nf)
        return np.lexsort((np.arange(nf), -s))[:k]
    m.select_blocks = select_blocks


def _m_bottom_k(m):
    def select_blocks(scores, k=m.TOPK):
        s = np.asarray(scores, np.float32).astype(np.float64)
        nf = s.shape[0]
        if nf <= k:
            return np.arange(nf)
        return np.sort(np.lexsort((np.arange(nf), s))[:k])
    m.select_blocks = select_blocks


def _m_drop_partial(m):
    orig = m.build_positions
    def build_positions(sel, L, kv_start, k=m.TOPK):
        return orig(sel, L - L % 4, kv_start, k)
    m.build_positions = build_positions


def _m_no_kv_offset(m):
    orig = m.build_positions
    def build_positions(sel, L, kv_start, k=m.TOPK):
        return orig(sel, L, 0, k)
    m.build_positions = build_positions


def _m_all_queries_full_length(m):
    m.query_length = lambda seq_len, nq, j: int(seq_len)


def _m_causal_off_by_one(m):
    m.query_length = lambda seq_len, nq, j: int(seq_len) - int(nq) + int(j)


def _m_ignore_scale(m):
    orig = m.sparse_attention
    m.sparse_attention = lambda qh, kr, vr, sm: orig(qh, kr, vr, 1.0)


def _m_gqa_modulo(m):
    def sparse_attention(q_heads, k_rows, v_rows, sm_scale):
        Hq, d = q_heads.shape
        Hkv = k_rows.shape[1]
        out = np.empty((Hq, d))
        for h in range(Hq):
            g = h % Hkv
            z = (k_rows[:, g, :] @ q_heads[h]) * sm_scale
            p = np.exp(z - z.max())
            out[h] = (p @ v_rows[:, g, :]) / p.sum()
        return out
    m.sparse_attention = sparse_attention


def _m_fp8_bias8(m):
    def fp8(codes):
        c = np.asarray(codes, np.uint8).astype(np.int64)
        s, e, mm = (c >> 7) & 1, (c >> 3) & 15, c & 7
        mag = np.where(e == 0, np.ldexp(mm / 8.0, -7), np.ldexp(1.0 + mm / 8.0, e - 8))
        mag = np.where((e == 15) & (mm == 7), np.nan, mag)
        return np.where(s == 1, -mag, mag)
    m.fp8_e4m3fn_to_f64 = fp8


def _m_fp8_no_subnormals(m):
    def fp8(codes):
        c = np.asarray(codes, np.uint8).astype(np.int64)
        s, e, mm = (c >> 7) & 1, (c >> 3) & 15, c & 7
        mag = np.ldexp(1.0 + mm / 8.0, e - 7)
        mag = np.where((e == 15) & (mm == 7), np.nan, mag)
        return np.where(s == 1, -mag, mag)
    m.fp8_e4m3fn_to_f64 = fp8


def _m_swap_kv_scales(m):
    orig = m.decode
    def decode(*a, **kw):
        a = list(a)
        a[10], a[11] = a[11], a[10]
        return orig(*a, **kw)
    m.decode = decode


def _m_score_sign(m):
    orig = m.block_scores
    m.block_scores = lambda iq, keys: -orig(iq, keys)


def _m_score_in_bf16(m):
    orig = m.block_scores
    def block_scores(iq, keys):
        s = orig(iq, keys)
        u = s.view(np.uint32) & np.uint32(0xFFFF0000)
        return u.view(np.float32)
    m.block_scores = block_scores


def _m_ignore_blk_start(m):
    orig = m.decode
    def decode(q_start, seq_len, kv_start, blk_start, *a, **kw):
        return orig(q_start, seq_len, kv_start, np.zeros_like(blk_start), *a, **kw)
    m.decode = decode


def _m_sel_pad_keeps_k(m):
    orig = m.select_blocks
    def select_blocks(scores, k=m.TOPK):
        got = orig(scores, k)
        return got[:-1] if got.shape[0] > 1 else got
    m.select_blocks = select_blocks


def _m_page_no_scale(m):
    orig = m.token_slots
    def token_slots(t, kv_start=0, page_row=None, page_size=None):
        if page_row is None:
            return orig(t, kv_start)
        t = np.asarray(t, dtype=np.int64)
        return np.asarray(page_row, np.int64)[t // page_size] + t % page_size
    m.token_slots = token_slots


def _m_reuse_keeps_all(m):
    def build_positions(sel, L, kv_start, k=m.TOPK, page_row=None, page_size=None):
        sel = np.asarray(sel, dtype=np.int64)
        nf = L // m.BLOCK
        full = (m.BLOCK * sel[:, None] + np.arange(m.BLOCK)[None, :]).reshape(-1)
        p = m.token_slots(np.concatenate([full, np.arange(m.BLOCK * nf, L)]), kv_start, page_row, page_size)
        out = np.full(m.BLOCK * k + m.BLOCK - 1, -1, dtype=np.int64)
        out[:p.shape[0]] = p
        return out, int(p.shape[0])
    m.build_positions = build_positions


def _m_compress_truncate(m):
    def bf16_bits_round_exact(value, negative_zero=False):
        if value == 0:
            return 0x8000 if negative_zero else 0
        bits = int(np.array([float(value)], np.float32).view(np.uint32)[0])
        return bits >> 16
    m.bf16_bits_round_exact = bf16_bits_round_exact


def _m_compress_ties_away(m):
    F = m.Fraction
    def bf16_bits_round_exact(value, negative_zero=False):
        neg = value < 0
        a = -value if neg else value
        if a == 0:
            return 0x8000 if negative_zero else 0
        e = int(np.frexp(float(a))[1]) - 1
        while F(2) ** e > a:
            e -= 1
        while F(2) ** (e + 1) <= a:
            e += 1
        unit = F(2) ** (max(e, -126) - 7)
        n = a / unit
        fl = n.numerator // n.denominator
        if n - fl >= F(1, 2):                       # ties away from zero
            fl += 1
        bits = int(np.array([float(fl * unit)], np.float32).view(np.uint32)[0]) >> 16
        return bits | (0x8000 if neg else 0)
    m.bf16_bits_round_exact = bf16_bits_round_exact


def _m_compress_first_block_off(m):
    orig = m.compress_new_keys
    def compress_new_keys(seq_len, prev_len, tok_keys, kv_start=0, page_row=None, page_size=None):
        return orig(seq_len, min(int(prev_len) + 4, int(seq_len)), tok_keys, kv_start, page_row, page_size)
    m.compress_new_keys = compress_new_keys


def _m_v_from_k(m):
    orig = m.sparse_attention
    m.sparse_attention = lambda qh, kr, vr, sm: orig(qh, kr, kr, sm)


def _m_softmax_unnormalised(m):
    def sparse_attention(q_heads, k_rows, v_rows, sm_scale):
        Hq, d = q_heads.shape
        G = Hq // k_rows.shape[1]
        out = np.empty((Hq, d))
        for h in range(Hq):
            z = (k_rows[:, h // G, :] @ q_heads[h]) * sm_scale
            out[h] = np.exp(z - z.max()) @ v_rows[:, h // G, :]
        return out
    m.sparse_attention = sparse_attention


def _m_block_index_not_scaled(m):
    def build_positions(sel, L, kv_start, k=m.TOPK, page_row=None, page_size=None):
        sel = np.asarray(sel, dtype=np.int64)
        nf = L // m.BLOCK
        sel = sel[sel < nf]
        full = (sel[:, None] + np.arange(m.BLOCK)[None, :]).reshape(-1)
        p = m.token_slots(np.concatenate([full, np.arange(m.BLOCK * nf, L)]), kv_start, page_row, page_size)
        out = np.full(m.BLOCK * k + m.BLOCK - 1, -1, dtype=np.int64)
        out[:p.shape[0]] = p
        return out, int(p.shape[0])
    m.build_positions = build_positions


def _m_partial_block_from_block_start(m):
    orig = m.build_positions
    def build_positions(sel, L, kv_start, k=m.TOPK, page_row=None, page_size=None):
        out, n = orig(sel, L, kv_start, k, page_row, page_size)
        pl = L % m.BLOCK
        if pl:
            nf = L // m.BLOCK
            out = out.copy()
            out[n - pl:n] = m.token_slots(np.arange(m.BLOCK * (nf - 1), m.BLOCK * (nf - 1) + pl) if nf else
                                          np.arange(pl) + 1, kv_start, page_row, page_size)
        return out, n
    m.build_positions = build_positions


def _m_page_row_of_first_request(m):
    orig = m.decode
    def decode(*a, **kw):
        if kw.get("page_table") is not None:
            pt = np.asarray(kw["page_table"])
            kw["page_table"] = np.repeat(pt[:1], pt.shape[0], axis=0)
        return orig(*a, **kw)
    m.decode = decode


def _m_kv_scales_ignored(m):
    orig = m.decode
    def decode(*a, **kw):
        a = list(a)
        if len(a) > 11 and a[10] is not None:
            a[10], a[11] = np.ones_like(a[10]), np.ones_like(a[11])
        for key in ("k_scale", "v_scale"):
            if kw.get(key) is not None:
                kw[key] = np.ones_like(kw[key])
        return orig(*a, **kw)
    m.decode = decode


MUTANTS = [_m_tie_higher_index, _m_unsorted_output, _m_bottom_k, _m_drop_partial, _m_no_kv_offset,
           _m_all_queries_full_length, _m_causal_off_by_one, _m_ignore_scale, _m_gqa_modulo,
           _m_fp8_bias8, _m_fp8_no_subnormals, _m_swap_kv_scales, _m_score_sign, _m_score_in_bf16,
           _m_ignore_blk_start, _m_sel_pad_keeps_k, _m_page_no_scale, _m_reuse_keeps_all,
           _m_compress_truncate, _m_compress_ties_away, _m_compress_first_block_off, _m_v_from_k,
           _m_softmax_unnormalised, _m_block_index_not_scaled, _m_partial_block_from_block_start,
           _m_page_row_of_first_request, _m_kv_scales_ignored]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__[3:])
def test_pins_catch_mutant(mutant):
    m = fresh_oracle()
    mutant(m)
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(m)
        except AssertionError:
            return
    pytest.fail(f"no pin caught mutant {mutant.__name__}")

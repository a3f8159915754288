"""Plain FP64 CPU oracle for the QSA decode path.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path and imports nothing from it.

What it computes follows the QSA selection-pipeline description in the
arex-research.com article on TokenSpeed serving Qwen3.8-Flash-Next, section
"稀疏选择、CuTe DSL 内核与 MTP 复用" (four optimisations), items 1-3:
  * tokens form 4-token micro-blocks, each full block has a compressed index key;
  * every query scores its full blocks into an FP32 buffer and keeps at most
    512 of them by top-k (at most 2,048 positions);
  * the current partial block is kept without selection, so the selection
    buffer has a fixed width of 2,051;
  * attention then runs over the gathered positions only, with BF16 queries
    and BF16 or FP8 E4M3 KV.
The 10100.com article (section on the first optimisation) describes the same
pipeline as: score the history, keep the relevant pieces, then find where they
sit in the cache.

Where the pages leave a step open, this file takes the plain reading:
  * block score = unscaled dot product of the 128-dim index query with the
    block's compressed key, exact sum rounded once to FP32;
  * top-k order = score descending, then block index ascending (the lower
    index wins ties); the selected set is reported in ascending block order;
  * MTP verify query j of a request with nq queries and cache length seq_len
    (verify tokens included) sees the causal prefix L = seq_len - nq + 1 + j;
    its full blocks are [0, L // 4) and its partial block is the last L % 4
    tokens (nothing is kept when L % 4 == 0);
  * a position is the physical KV slot of the token: kv_start + token index,
    or, with a paged cache, page_table[token // page_size] * page_size +
    token % page_size (page_size a multiple of 4);
  * a selection reused at another length keeps only its blocks that are full
    for the new query (later MTP draft steps reuse earlier positions: 10100.com
    article, section on the third optimisation);
  * the compressed key of a block (the pages do not give the rule) is the mean
    of its four per-token index keys, rounded once to BF16, nearest-even;
  * softmax scale is passed in (1/sqrt(128) for head_dim 128); GQA maps query
    head h to KV head h // (Hq / Hkv);
  * FP8 is OCP E4M3FN with one FP32 scale per KV head for K and one for V.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

BLOCK = 4                              # tokens per micro-block
TOPK = 512                             # at most this many full blocks per query
WIDTH = BLOCK * TOPK + BLOCK - 1       # 2,051: selected positions + partial block


def bf16_to_f64(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64.  BF16 is the top half of an FP32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def fp8_e4m3fn_to_f64(codes) -> np.ndarray:
    """OCP FP8 E4M3FN bytes -> float64.

    Layout s.eeee.mmm with exponent bias 7; e == 0 encodes subnormals
    (m/8) * 2^-6; there are no infinities and s.1111.111 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def query_length(seq_len: int, nq: int, j: int) -> int:
    """Causal prefix length of verify query j (0-based) of a request with nq queries."""
    return int(seq_len) - int(nq) + 1 + int(j)


def block_scores(idx_q_bits, key_bits) -> np.ndarray:
    """FP32 score of one query against each full block's compressed key.

    idx_q_bits: uint16[128] BF16 index query; key_bits: uint16[nf, 128] keys.
    The dot product is taken in float64 and rounded once to float32.
    """
    keys = bf16_to_f64(key_bits).reshape(-1, bf16_to_f64(idx_q_bits).shape[0])
    return (keys @ bf16_to_f64(idx_q_bits)).astype(np.float32)


def select_blocks(scores, k: int = TOPK) -> np.ndarray:
    """Indices of the kept full blocks, ascending.

    If there are at most k blocks all are kept.  Otherwise the k blocks that
    come first when ordered by (score descending, index ascending) are kept.
    +0.0 and -0.0 compare equal.
    """
    s = np.asarray(scores, dtype=np.float32).astype(np.float64)
    nf = s.shape[0]
    if nf <= k:
        return np.arange(nf, dtype=np.int64)
    order = np.lexsort((np.arange(nf), -s))     # primary key last: -score, then index
    return np.sort(order[:k]).astype(np.int64)


def token_slots(t, kv_start: int = 0, page_row=None, page_size: int | None = None) -> np.ndarray:
    """Physical KV slots of logical token indices t of one request."""
    t = np.asarray(t, dtype=np.int64)
    if page_row is None:
        return t + int(kv_start)
    page_row = np.asarray(page_row, dtype=np.int64)
    return page_row[t // page_size] * page_size + t % page_size


def build_positions(sel, L: int, kv_start: int, k: int = TOPK, page_row=None, page_size: int | None = None):
    """Fixed-width position buffer of one query and its valid length.

    Each kept block b that is full for this query (b < L // 4) contributes the
    slots of its tokens 4b..4b+3, in block order; the partial block's tokens
    [4 * (L // 4), L) follow; the rest of the 4k+3 entries is -1.
    """
    sel = np.asarray(sel, dtype=np.int64)
    nf = L // BLOCK
    sel = sel[(sel >= 0) & (sel < nf)]
    full = (BLOCK * sel[:, None] + np.arange(BLOCK)[None, :]).reshape(-1)
    partial = np.arange(BLOCK * nf, L, dtype=np.int64)
    p = token_slots(np.concatenate([full, partial]), kv_start, page_row, page_size)
    width = BLOCK * k + BLOCK - 1
    out = np.full(width, -1, dtype=np.int64)
    out[:p.shape[0]] = p
    return out, int(p.shape[0])


BF16_MAX = Fraction(2 - Fraction(1, 128)) * Fraction(2) ** 127


def bf16_bits_round_exact(value: Fraction, negative_zero: bool = False) -> int:
    """BF16 bit pattern of an exact rational, rounded to nearest, ties to even
    (IEEE round-to-nearest: beyond the largest finite value it becomes inf).

    A BF16 number is s * m * 2^(e-7) with an 8-bit significand m in [128, 256)
    for normal values (e >= -126) and the fixed unit 2^-133 below 2^-126; the
    value is divided by the unit of its binade, rounded half-to-even to an
    integer and scaled back.  A zero result is -0 only when negative_zero.
    """
    neg = value < 0
    a = -value if neg else value
    if a == 0:
        return 0x8000 if negative_zero else 0x0000
    e = int(np.frexp(float(a))[1]) - 1
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    unit = Fraction(2) ** (e - 7)
    n = a / unit
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * unit
    if r > BF16_MAX:
        bits = 0x7F80
    else:
        bits = int(np.array([float(r)], dtype=np.float32).view(np.uint32)[0]) >> 16
    return bits | (0x8000 if neg else 0)


def compress_block_key(token_key_bits) -> np.ndarray:
    """Compressed index key of one 4-token block from its tokens' BF16 keys.

    token_key_bits: uint16 [4, d].  Each dimension is the exact mean of the
    four values, rounded once to BF16 (nearest, ties to even); a zero mean is
    -0 only when all four values are -0 (as an IEEE sum in token order gives).
    """
    bits = np.asarray(token_key_bits, dtype=np.uint16)
    vals = bf16_to_f64(bits)
    out = np.empty(bits.shape[1], dtype=np.uint16)
    for dd in range(bits.shape[1]):
        total = sum(Fraction(float(v)) for v in vals[:, dd])
        all_neg_zero = bool(np.all(bits[:, dd] == 0x8000))
        out[dd] = bf16_bits_round_exact(total / 4, negative_zero=all_neg_zero)
    return out


def compress_new_keys(seq_len: int, prev_len: int, tok_keys, kv_start: int = 0, page_row=None,
                      page_size: int | None = None) -> dict:
    """Keys of the blocks completed by the tokens appended since prev_len:
    {block index b: uint16 [d]} for every b with prev_len <= 4b + 3 < seq_len."""
    out = {}
    prev_len = min(max(int(prev_len), 0), int(seq_len))
    for b in range(prev_len // BLOCK, int(seq_len) // BLOCK):
        slots = token_slots(np.arange(BLOCK * b, BLOCK * b + BLOCK), kv_start, page_row, page_size)
        out[b] = compress_block_key(np.asarray(tok_keys)[slots])
    return out


def sparse_attention(q_heads, k_rows, v_rows, sm_scale: float) -> np.ndarray:
    """Softmax attention of each query head over gathered rows only.

    q_heads: float64 [Hq, d]; k_rows, v_rows: float64 [n, Hkv, d] (already
    dequantised).  Query head h reads KV head h // (Hq / Hkv).
    """
    Hq, d = q_heads.shape
    Hkv = k_rows.shape[1]
    G = Hq // Hkv
    out = np.empty((Hq, d), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        z = (k_rows[:, g, :] @ q_heads[h]) * sm_scale
        p = np.exp(z - z.max())
        out[h] = (p @ v_rows[:, g, :]) / p.sum()
    return out


def _dequant(cache, rows, kv_dtype, scale):
    if kv_dtype == "bf16":
        return bf16_to_f64(cache[rows])
    if kv_dtype == "fp8_e4m3":
        return fp8_e4m3fn_to_f64(cache[rows]) * np.asarray(scale, np.float64)[None, :, None]
    raise ValueError(kv_dtype)


def decode(q_start, seq_len, kv_start, blk_start, idx_q, ckeys, q, k_cache, v_cache,
           kv_dtype: str, k_scale=None, v_scale=None, k: int = TOPK, sm_scale: float | None = None,
           want_scores: bool = True, queries=None, page_table=None, page_size: int | None = None) -> dict:
    """Run score -> top-k -> positions -> gather attention for every query.

    Returns a dict with per-query 'scores' (list of float32 arrays, if asked),
    'sel' int32 [num_q, k] (-1 padded), 'n_sel', 'pos' int32 [num_q, 4k+3]
    (-1 padded), 'n_pos', and 'out' float64 [num_q, Hq, d].  `queries` limits
    the work to a subset of query indices (other rows stay zero / -1).
    With page_table ([num_req][pages] int) and page_size, token slots go
    through the page table instead of kv_start.
    """
    q_start = np.asarray(q_start, np.int64)
    num_q = int(q_start[-1])
    Hq, d = q.shape[1], q.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    width = BLOCK * k + BLOCK - 1
    res = {
        "scores": [None] * num_q,
        "sel": np.full((num_q, k), -1, np.int32),
        "n_sel": np.zeros(num_q, np.int32),
        "pos": np.full((num_q, width), -1, np.int32),
        "n_pos": np.zeros(num_q, np.int32),
        "out": np.zeros((num_q, Hq, d), np.float64),
    }
    wanted = None if queries is None else set(int(x) for x in queries)
    for r in range(len(seq_len)):
        nq = int(q_start[r + 1] - q_start[r])
        for j in range(nq):
            qi = int(q_start[r]) + j
            if wanted is not None and qi not in wanted:
                continue
            L = query_length(seq_len[r], nq, j)
            nf = L // BLOCK
            b0 = int(blk_start[r])
            s = block_scores(idx_q[qi], ckeys[b0:b0 + nf])
            sel = select_blocks(s, k)
            if page_table is None:
                pos, n_pos = build_positions(sel, L, int(kv_start[r]), k)
            else:
                pos, n_pos = build_positions(sel, L, 0, k, page_table[r], page_size)
            rows = pos[:n_pos]
            kr = _dequant(k_cache, rows, kv_dtype, k_scale)
            vr = _dequant(v_cache, rows, kv_dtype, v_scale)
            res["out"][qi] = sparse_attention(bf16_to_f64(q[qi]), kr, vr, sm_scale)
            if want_scores:
                res["scores"][qi] = s
            res["sel"][qi, :sel.shape[0]] = sel
            res["n_sel"][qi] = sel.shape[0]
            res["pos"][qi] = pos
            res["n_pos"][qi] = n_pos
    return res

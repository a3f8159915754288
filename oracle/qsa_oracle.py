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
  * a position is the physical KV slot kv_start + token index;
  * softmax scale is passed in (1/sqrt(128) for head_dim 128); GQA maps query
    head h to KV head h // (Hq / Hkv);
  * FP8 is OCP E4M3FN with one FP32 scale per KV head for K and one for V.
"""
from __future__ import annotations

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


def build_positions(sel, L: int, kv_start: int, k: int = TOPK):
    """Fixed-width position buffer of one query and its valid length.

    Each kept block b contributes its four slots 4b..4b+3, in block order; the
    partial block [4 * (L // 4), L) follows; the rest of the 4k+3 entries is -1.
    Slots are offset by the request's first KV slot.
    """
    sel = np.asarray(sel, dtype=np.int64)
    nf = L // BLOCK
    full = (BLOCK * sel[:, None] + np.arange(BLOCK)[None, :]).reshape(-1)
    partial = np.arange(BLOCK * nf, L, dtype=np.int64)
    p = np.concatenate([full, partial]) + int(kv_start)
    width = BLOCK * k + BLOCK - 1
    out = np.full(width, -1, dtype=np.int64)
    out[:p.shape[0]] = p
    return out, int(p.shape[0])


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
           want_scores: bool = True, queries=None) -> dict:
    """Run score -> top-k -> positions -> gather attention for every query.

    Returns a dict with per-query 'scores' (list of float32 arrays, if asked),
    'sel' int32 [num_q, k] (-1 padded), 'n_sel', 'pos' int32 [num_q, 4k+3]
    (-1 padded), 'n_pos', and 'out' float64 [num_q, Hq, d].  `queries` limits
    the work to a subset of query indices (other rows stay zero / -1).
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
            pos, n_pos = build_positions(sel, L, int(kv_start[r]), k)
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

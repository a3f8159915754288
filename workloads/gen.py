"""Seeded synthetic workloads for QSA block-sparse decode attention.

Shapes follow the serving setup the pages describe: 4-token micro-blocks with
one 128-dim compressed index key per full block, up to 4 MTP verify queries
per request, BF16 queries, BF16 or FP8 E4M3 KV cache, and SWE-Smith-like
context lengths (a 50,000-token first turn, +800 tokens per turn).  No data
from any benchmark is used: only these shapes.

Everything here is random-number generation plus storage encoding.  Arrays are
returned as raw bit patterns (uint16 for BF16, uint8 for FP8 E4M3FN) so the
oracle and the GPU read byte-identical inputs.

Draw order (fixed, one PCG64 stream per workload):
  1. lengths, queries per request, layout gaps
  2. index queries   3. compressed keys   4. attention queries
  5. K cache         6. V cache
Normal N(0,1) values are realised as 16-bit uniform draws mapped through the
65,536-point inverse normal CDF (mid-quantiles), then rounded to BF16 or
scaled and rounded to FP8.  Integer index values are uniform in [-8, 8].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

INDEX_DIM = 128
HEAD_DIM = 128
FP8_E4M3FN_MAX = 448.0

_QTABLE = None


def normal_quantile_table() -> np.ndarray:
    """float32[65536]: inverse standard normal CDF at (i + 0.5) / 65536."""
    global _QTABLE
    if _QTABLE is None:
        from scipy.special import ndtri
        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _QTABLE = ndtri(p).astype(np.float32)
    return _QTABLE


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to BF16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def fp8_e4m3fn_bits_from_f32(x) -> np.ndarray:
    """Encode float32 values as OCP FP8 E4M3FN bytes (RNE, saturating at +-448)."""
    import torch
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32),
                                 -FP8_E4M3FN_MAX, FP8_E4M3FN_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


@dataclass
class Workload:
    """One batch of decode / MTP-verify queries and the caches they read.

    Request r owns queries [q_start[r], q_start[r+1]), a contiguous KV region
    starting at slot kv_start[r] holding seq_len[r] tokens (this step's verify
    tokens included), and compressed-key rows starting at blk_start[r], one per
    full 4-token block of those seq_len[r] tokens.
    """
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    kv_dtype: str                      # "bf16" or "fp8_e4m3"
    q_start: np.ndarray                # int32 [B+1]
    seq_len: np.ndarray                # int32 [B]
    kv_start: np.ndarray               # int32 [B]
    blk_start: np.ndarray              # int32 [B]
    idx_q: np.ndarray                  # uint16 [num_q, 128]   BF16 bits
    ckeys: np.ndarray                  # uint16 [rows, 128]    BF16 bits
    q: np.ndarray                      # uint16 [num_q, Hq, 128] BF16 bits
    k_cache: np.ndarray                # uint16|uint8 [slots, Hkv, 128]
    v_cache: np.ndarray
    k_scale: np.ndarray | None = None  # float32 [Hkv] (FP8 only)
    v_scale: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def num_req(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def num_q(self) -> int:
        return int(self.q_start[-1])

    @property
    def key_rows(self) -> int:
        return int(self.ckeys.shape[0])

    @property
    def kv_slots(self) -> int:
        return int(self.k_cache.shape[0])

    def queries_of(self, r: int) -> range:
        return range(int(self.q_start[r]), int(self.q_start[r + 1]))


def _int_bf16(rng, shape) -> np.ndarray:
    vals = rng.integers(-8, 9, size=shape, dtype=np.int8)
    return bf16_bits_from_f32(vals.astype(np.float32))


def _normal_u16(rng, shape) -> np.ndarray:
    return rng.integers(0, 65536, size=shape, dtype=np.uint16)


def _kv_from_u16(u: np.ndarray, kv_dtype: str, num_kv_heads: int):
    table = normal_quantile_table()
    if kv_dtype == "bf16":
        return bf16_bits_from_f32(table)[u], None
    if kv_dtype != "fp8_e4m3":
        raise ValueError(kv_dtype)
    codes = np.empty(u.shape, dtype=np.uint8)
    scale = np.empty(num_kv_heads, dtype=np.float32)
    for g in range(num_kv_heads):
        ug = u[:, g, :]
        amax = max(abs(float(table[int(ug.min())])), abs(float(table[int(ug.max())])))
        scale[g] = np.float32(amax / FP8_E4M3FN_MAX)
        head_table = fp8_e4m3fn_bits_from_f32(table / scale[g])
        codes[:, g, :] = head_table[ug]
    return codes, scale


def make_custom(name: str, seq_lens, nq_per_req, num_q_heads: int, num_kv_heads: int,
                kv_dtype: str = "bf16", seed: int = 0, index_values: str = "int",
                tie_fraction: float | None = None, gaps: bool = True,
                rng: np.random.Generator | None = None) -> Workload:
    """Build a workload from explicit per-request lengths and query counts.

    index_values: "int"  -> index query and keys uniform integers in [-8, 8]
                  "normal" -> N(0,1) rounded to BF16
    tie_fraction: if set (integer index values only), a random subset of that
                  fraction of each request's blocks gets the key 8*s, where the
                  index queries are s * u with s a random sign vector and u
                  uniform in {1..8}; those blocks then share the strict maximum
                  score for every query of the request.
    gaps: leave a few random unused slots / key rows before each request.
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    nq = np.asarray(nq_per_req, dtype=np.int64)
    B = seq_lens.shape[0]
    assert nq.shape == (B,) and B >= 1
    assert np.all(seq_lens >= 1) and np.all(nq >= 1) and np.all(nq <= 4) and np.all(nq <= seq_lens)

    # 1. layout
    kv_gap = rng.integers(0, 8, size=B) if gaps else np.zeros(B, np.int64)
    blk_gap = rng.integers(0, 4, size=B) if gaps else np.zeros(B, np.int64)
    nblk = seq_lens // 4
    kv_start = np.zeros(B, np.int64)
    blk_start = np.zeros(B, np.int64)
    kv_off = blk_off = 0
    for r in range(B):
        kv_off += int(kv_gap[r]); kv_start[r] = kv_off; kv_off += int(seq_lens[r])
        blk_off += int(blk_gap[r]); blk_start[r] = blk_off; blk_off += int(nblk[r])
    slots = kv_off + (3 if gaps else 0)
    rows = max(blk_off, 1)
    q_start = np.concatenate([[0], np.cumsum(nq)])
    num_q = int(q_start[-1])
    assert slots < 2**31 and rows < 2**31

    # 2-3. index queries and compressed keys
    if index_values == "normal":
        table_bf16 = bf16_bits_from_f32(normal_quantile_table())
        idx_q = table_bf16[_normal_u16(rng, (num_q, INDEX_DIM))]
        ckeys = table_bf16[_normal_u16(rng, (rows, INDEX_DIM))]
    elif index_values == "int":
        if tie_fraction is None:
            idx_q = _int_bf16(rng, (num_q, INDEX_DIM))
            ckeys = _int_bf16(rng, (rows, INDEX_DIM))
        else:
            idx_q = np.empty((num_q, INDEX_DIM), np.uint16)
            ckeys = _int_bf16(rng, (rows, INDEX_DIM))
            tie_sets = []
            for r in range(B):
                s = rng.choice(np.array([-1, 1], np.int64), size=INDEX_DIM)
                for qi in range(int(q_start[r]), int(q_start[r + 1])):
                    u = rng.integers(1, 9, size=INDEX_DIM)
                    idx_q[qi] = bf16_bits_from_f32((s * u).astype(np.float32))
                n_tie = int(math.ceil(tie_fraction * int(nblk[r])))
                tie = np.sort(rng.choice(int(nblk[r]), size=n_tie, replace=False)) if n_tie else \
                    np.zeros(0, np.int64)
                kstar = bf16_bits_from_f32((8 * s).astype(np.float32))
                base = int(blk_start[r])
                # keys outside the tie set must differ from k*
                seg = ckeys[base:base + int(nblk[r])]
                clash = np.all(seg == kstar[None, :], axis=1)
                while clash.any():
                    seg[clash] = _int_bf16(rng, (int(clash.sum()), INDEX_DIM))
                    clash = np.all(seg == kstar[None, :], axis=1)
                seg[tie] = kstar[None, :]
                tie_sets.append(tie)
    else:
        raise ValueError(index_values)

    # 4. attention queries
    table_bf16 = bf16_bits_from_f32(normal_quantile_table())
    q = table_bf16[_normal_u16(rng, (num_q, num_q_heads, HEAD_DIM))]

    # 5-6. KV cache
    k_u = _normal_u16(rng, (slots, num_kv_heads, HEAD_DIM))
    k_cache, k_scale = _kv_from_u16(k_u, kv_dtype, num_kv_heads)
    del k_u
    v_u = _normal_u16(rng, (slots, num_kv_heads, HEAD_DIM))
    v_cache, v_scale = _kv_from_u16(v_u, kv_dtype, num_kv_heads)
    del v_u

    meta = {}
    if tie_fraction is not None and index_values == "int":
        meta["tie_sets"] = tie_sets
    return Workload(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    kv_dtype=kv_dtype, q_start=q_start.astype(np.int32),
                    seq_len=seq_lens.astype(np.int32), kv_start=kv_start.astype(np.int32),
                    blk_start=blk_start.astype(np.int32), idx_q=idx_q, ckeys=ckeys, q=q,
                    k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale, meta=meta)


# The five named workloads.  Each is a function of its seed only.
CONFIGS = {
    # one request, one decode query, 8,192-token context, 16 q heads / 2 KV heads, BF16
    "single8k": dict(seed=101, heads=(16, 2), kv="bf16"),
    # one request, 4 MTP verify queries, 50,000-token context, 32 / 4 heads, BF16
    "mtp50k": dict(seed=102, heads=(32, 4), kv="bf16"),
    # 32 requests x 4 verify queries, 50,000 + 800 t tokens (t uniform 0..14), FP8 E4M3 KV
    "mtp50k_b32_fp8": dict(seed=103, heads=(32, 4), kv="fp8_e4m3"),
    # one request, 4 verify queries, 262,144 tokens, ~5% of blocks tied at the top score
    "mtp262k_ties": dict(seed=104, heads=(32, 4), kv="bf16"),
    "mtp262k_ties_fp8": dict(seed=104, heads=(32, 4), kv="fp8_e4m3"),
    # 64 requests, lengths log-uniform in [1, 131072], 1 or 4 queries each, 16 / 2 heads
    "ragged64": dict(seed=105, heads=(16, 2), kv="bf16"),
    # one request, 4 verify queries, a 1,048,576-token context (262,144 blocks), 32 / 4 heads, BF16
    "mtp1m": dict(seed=106, heads=(32, 4), kv="bf16"),
}


def make_workload(name: str) -> Workload:
    cfg = CONFIGS[name]
    seed = cfg["seed"]
    hq, hkv = cfg["heads"]
    rng = np.random.Generator(np.random.PCG64(seed))
    tie = None
    if name == "single8k":
        lens, nq = [8192], [1]
    elif name == "mtp50k":
        lens, nq = [50000], [4]
    elif name == "mtp50k_b32_fp8":
        t = rng.integers(0, 15, size=32)
        lens, nq = (50000 + 800 * t).tolist(), [4] * 32
    elif name.startswith("mtp262k_ties"):
        lens, nq, tie = [262144], [4], 0.05
    elif name == "mtp1m":
        lens, nq = [1 << 20], [4]
    elif name == "ragged64":
        u = rng.random(64)
        lens = np.clip(np.floor(np.exp(u * math.log(131072.0))), 1, 131072).astype(np.int64)
        nq = np.where(rng.random(64) < 0.5, 1, 4)
        nq = np.minimum(nq, lens)
    else:
        raise KeyError(name)
    return make_custom(name, lens, nq, hq, hkv, kv_dtype=cfg["kv"], seed=seed,
                       tie_fraction=tie, rng=rng)


def paged_layout(w, page_size: int, seed: int):
    """The workload's caches re-laid out in pages of page_size tokens placed at a
    random permutation of physical pages, with the page table that maps them."""
    rng = np.random.default_rng(seed)
    seq = [int(x) for x in w.seq_len]
    pages = [-(-s // page_size) for s in seq]
    ppr = max(pages)
    perm = rng.permutation(sum(pages))
    table = np.zeros((len(seq), ppr), np.int64)
    kc = np.zeros((sum(pages) * page_size,) + w.k_cache.shape[1:], w.k_cache.dtype)
    vc = np.zeros_like(kc)
    nxt = 0
    for r, s in enumerate(seq):
        for p in range(pages[r]):
            phys = int(perm[nxt]); nxt += 1
            table[r, p] = phys
            lo, hi = p * page_size, min(s, (p + 1) * page_size)
            src = int(w.kv_start[r]) + np.arange(lo, hi)
            dst = phys * page_size + np.arange(hi - lo)
            kc[dst], vc[dst] = w.k_cache[src], w.v_cache[src]
    return table, kc, vc

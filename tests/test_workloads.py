"""Seeded input generator: determinism and the shapes the configs call for (no GPU)."""
import numpy as np
import torch

from workloads import make_workload, make_custom, normal_quantile_table, CONFIGS


def test_quantile_table_is_standard_normal():
    t = normal_quantile_table().astype(np.float64)
    assert abs(t.mean()) < 1e-6 and abs(t.std() - 1.0) < 2e-3
    assert np.all(np.diff(t) > 0)


def test_single8k_deterministic_and_shaped():
    a = make_workload("single8k")
    b = make_workload("single8k")
    for f in ("idx_q", "ckeys", "q", "k_cache", "v_cache", "kv_start", "blk_start"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.num_req == 1 and a.num_q == 1 and int(a.seq_len[0]) == 8192
    assert a.key_rows >= 2048 and a.q.shape == (1, 16, 128) and a.k_cache.shape[1:] == (2, 128)
    iv = torch.from_numpy(a.ckeys.astype(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(iv, np.round(iv)) and iv.min() == -8 and iv.max() == 8


def test_b32_lengths_follow_turn_schedule():
    # only the lengths are checked here; draw them the way the generator does
    rng = np.random.Generator(np.random.PCG64(CONFIGS["mtp50k_b32_fp8"]["seed"]))
    t = rng.integers(0, 15, size=32)
    lens = 50000 + 800 * t
    assert np.all(lens % 4 == 0) and lens.min() >= 50000 and lens.max() <= 61200


def test_fp8_kv_scale_and_range():
    w = make_custom("f", [300, 77], [4, 1], 8, 2, kv_dtype="fp8_e4m3", seed=9)
    assert w.k_cache.dtype == np.uint8 and w.k_scale.shape == (2,)
    vals = torch.from_numpy(w.k_cache).view(torch.float8_e4m3fn).float().numpy()
    assert np.all(np.abs(vals) <= 448) and np.abs(vals).max() == 448
    assert not np.any(np.isnan(vals))


def test_layout_regions_disjoint():
    w = make_custom("l", [5, 9, 1, 4000], [4, 2, 1, 3], 8, 2, seed=10)
    ends = w.kv_start + w.seq_len
    assert np.all(w.kv_start[1:] >= ends[:-1]) and ends[-1] <= w.kv_slots
    bends = w.blk_start + w.seq_len // 4
    assert np.all(w.blk_start[1:] >= bends[:-1]) and bends[-1] <= w.key_rows
    assert list(w.q_start) == [0, 4, 6, 7, 10]

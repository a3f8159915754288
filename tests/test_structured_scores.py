"""The fused decode path on index keys laid out so that the best blocks of a
row crowd together: scores rising or falling with the block index (whole
64-block groups win), a few hot groups scattered over the row, and one flat
row where every block ties (the lowest indices win).  At 50,000 tokens and on
a mixed FP8 batch up to 131,075 tokens, the selection must equal the oracle's
bit for bit and the output must be within 2e-3 * max|out|."""
import numpy as np
import pytest

from workloads import bf16_bits_from_f32, make_custom
from workloads.device import upload
from gpu_helpers import (assert_lean_decode_same, assert_out_close, assert_selection_equal, need_gpu, oracle_decode,
                         run_decode, say)

pytestmark = pytest.mark.gpu


def _structured(w, pattern: str, seed: int):
    """Overwrite the index queries and compressed keys so that each request's
    block score follows `pattern` (all values small integers: exact BF16
    inputs and exact FP32 scores)."""
    rng = np.random.default_rng(seed)
    iq = np.zeros((w.num_q, 128), np.float32)
    iq[:, 0], iq[:, 1], iq[:, 2] = 16.0, 1.0, 1.0
    w.idx_q[:] = bf16_bits_from_f32(iq)
    for r in range(w.num_req):
        nblk = int(w.seq_len[r]) // 4
        b = np.arange(nblk)
        g = b // 64
        ck = np.zeros((nblk, 128), np.float32)
        if pattern == "rising":            # score = group index: the last groups win whole
            lvl = g
        elif pattern == "falling":         # the first groups win whole
            lvl = g.max() - g
        elif pattern == "hot_groups":      # a few scattered groups far above the rest
            lvl = rng.integers(0, 8, nblk)
            hot = rng.choice(g.max() + 1, size=min(12, g.max() + 1), replace=False)
            lvl[np.isin(g, hot)] += 200
        elif pattern == "flat":            # every block ties: the lowest indices win
            lvl = np.zeros(nblk, np.int64)
        else:
            raise ValueError(pattern)
        ck[:, 0], ck[:, 1] = lvl // 16, lvl % 16
        if pattern == "hot_groups":        # break ties inside groups in a random order
            ck[:, 2] = rng.integers(0, 4, nblk)
        w.ckeys[int(w.blk_start[r]):int(w.blk_start[r]) + nblk] = bf16_bits_from_f32(ck)
    return w


@pytest.mark.parametrize("pattern", ["rising", "falling", "hot_groups", "flat"])
@pytest.mark.parametrize("shape", ["50k", "mixed"])
def test_decode_saturated_groups(pattern, shape):
    need_gpu()
    if shape == "50k":
        w = make_custom(f"sat-{pattern}", [50000], [4], 32, 4, seed=1101)
    else:
        w = make_custom(f"sat-{pattern}-mixed", [2049, 2300, 9001, 20000, 65536, 131072 + 3], [4, 1, 3, 4, 2, 4],
                        16, 2, kv_dtype="fp8_e4m3", seed=1102)
    w = _structured(w, pattern, seed=1103)
    say("qsa_decode saturated groups", w.name, "queries", w.num_q)
    ref = oracle_decode(w, want_scores=False)
    dev = upload(w)
    got = run_decode(w, dev)
    assert_selection_equal(got, ref)
    assert_out_close(got["out"], ref["out"])
    assert_lean_decode_same(w, got, dev)

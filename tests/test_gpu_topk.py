"""GPU parity of the standalone selector (topk_select) against the oracle's
full sort.  Selection over identical fp32 inputs is integer work: the sets
and the returned values must match exactly."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

import dsa_lightning_indexer_03_amd as dsa  # noqa: E402
from oracle import indexer  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(scores, K, row_len=None):
    idx, val = dsa.topk_select(dev(scores), K, row_len=None if row_len is None else dev(row_len))
    torch.cuda.synchronize()
    return host(idx), host(val)


def compare(scores, K, row_len=None, name=""):
    say(f"topk_select {name}: rows={scores.shape[0]} cols={scores.shape[1]} K={K}")
    gi, gv = run(scores, K, row_len)
    oi, ov = indexer.topk_rows(scores, row_len, K)
    for r in range(scores.shape[0]):
        n = scores.shape[1] if row_len is None else int(row_len[r])
        m = min(K, n)
        assert np.all(gi[r, m:] == -1) and np.all(np.isneginf(gv[r, m:])), (name, r)
        assert sorted(gi[r, :m].tolist()) == sorted(oi[r, :m].tolist()), (name, r)
        # values are the input scores of the returned positions (-0.0 == +0.0)
        assert np.array_equal(gv[r, :m], scores[r, gi[r, :m]]), (name, r)


def test_random_rows():
    rng = np.random.default_rng(100)
    compare(rng.standard_normal((8, 5000)).astype(np.float32), 100, name="random")


def test_row_lengths_including_empty_and_short():
    rng = np.random.default_rng(101)
    s = rng.standard_normal((7, 3000)).astype(np.float32)
    rl = np.array([0, 1, 99, 100, 101, 2999, 3000], np.int32)
    compare(s, 100, rl, name="row_len")


def test_tie_heavy_rows():
    rng = np.random.default_rng(102)
    s = np.round(rng.standard_normal((6, 20000)), 1).astype(np.float32)
    compare(s, 2048, name="ties")


def test_signed_zeros_tie():
    rng = np.random.default_rng(103)
    s = rng.choice(np.array([-0.0, 0.0, 0.0, 1.0, -1.0], np.float32), size=(4, 9000)).astype(np.float32)
    compare(s, 2048, name="zeros")


def test_huge_exact_tie_uses_lowest_positions():
    s = np.ones((2, 40000), np.float32)
    s[1, 5] = 2.0
    gi, _ = run(s, 2048)
    assert sorted(gi[0].tolist()) == list(range(2048))
    assert sorted(gi[1].tolist()) == list(range(2048))
    compare(s, 2048, name="huge tie")


def test_crowded_bin_beyond_lds():
    rng = np.random.default_rng(104)
    s = rng.standard_normal((3, 60000)).astype(np.float32)
    s[:, ::2] = 0.75 + rng.integers(0, 4, size=(3, 30000)).astype(np.float32) * 1e-6
    compare(s, 2048, name="crowded")


def test_long_rows_and_infinities():
    rng = np.random.default_rng(105)
    s = rng.standard_normal((4, 131072)).astype(np.float32)
    s[0, :100000] = -np.inf
    s[1, ::3] = -np.inf
    compare(s, 2048, name="long")


def test_all_k_values_small():
    rng = np.random.default_rng(106)
    s = rng.standard_normal((3, 777)).astype(np.float32)
    for K in (1, 2, 7, 64, 776, 777, 778, 2048):
        compare(s, K, name=f"K={K}")


def test_strided_rows_and_positive_infinity():
    """Rows read from a wider matrix (row stride 7001 floats, first column at
    offset 3): +inf entries rank first; a row holding more +inf entries than
    k keeps the lowest positions among them."""
    rng = np.random.default_rng(107)
    wide = rng.standard_normal((5, 7001)).astype(np.float32)
    wide[0, 3 + np.arange(0, 6000, 700)] = np.inf          # fewer than k
    wide[1, 3:3 + 6000:2] = np.inf                          # 3000 > k
    wide[2, 3 + np.array([5, 6, 5999])] = [np.inf, -np.inf, np.inf]
    view = dev(wide)[:, 3:6003]
    assert view.stride(0) == 7001 and not view.is_contiguous()
    K = 1000
    say(f"topk_select strided: rows=5 cols=6000 row_stride=7001 K={K}")
    idx, val = dsa.topk_select(view, K)
    torch.cuda.synchronize()
    gi, gv = host(idx), host(val)
    s = wide[:, 3:6003]
    oi, _ = indexer.topk_rows(s, None, K)
    for r in range(5):
        assert sorted(gi[r].tolist()) == sorted(oi[r].tolist()), r
        assert np.array_equal(gv[r], s[r, gi[r]]), r
    assert sorted(gi[1].tolist()) == list(range(0, 2 * K, 2))


def test_maximum_columns():
    """Rows of the largest supported length (4194304 columns), one of them
    cut short by its row length; k = 2048."""
    rng = np.random.default_rng(108)
    s = rng.standard_normal((2, 4194304)).astype(np.float32)
    s[1, 4194000:] = 100.0  # past row 1's length: never selected
    compare(s, 2048, np.array([4194304, 4194000], np.int32), name="max cols")

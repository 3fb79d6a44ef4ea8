"""GPU checks of the short-row bypass: when no score is requested, blocks of
rows with at most k valid positions skip scoring and return positions
0 .. t, then -1.  Their output must be identical to the scored path's, and
every other row too."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_03_amd as dsa
import synth
from gpu_util import dev, host, say
from oracle import indexer
from oracle.check import check_topk_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def prefill_idx(inp, K, want_topk_score):
    idx, _, _ = dsa.indexer_prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), K,
                                    q_scale=dev(inp.get("q_scale")), k_scale=dev(inp.get("k_scale")),
                                    want_topk_score=want_topk_score)
    torch.cuda.synchronize()
    return host(idx)


@pytest.mark.parametrize("dtype,L,K,H", [("fp8", 5000, 2048, 64), ("bf16", 5000, 2048, 64), ("fp8", 300, 512, 64),
                                         ("bf16", 1000, 64, 64), ("fp8", 3000, 2048, 48), ("bf16", 3000, 2048, 48)])
def test_bypass_equals_scored_path(dtype, L, K, H):
    inp = synth.prefill_inputs(1, L, H, 128, dtype, seed=950 + L + K + H)
    say(f"bypass {dtype} L={L} K={K} H={H}")
    fast = prefill_idx(inp, K, want_topk_score=False)
    full = prefill_idx(inp, K, want_topk_score=True)
    # the order inside a row is unspecified (a block that scores its sampled
    # chunks first lists them first): compare each row as a set
    assert np.array_equal(np.sort(fast, axis=2), np.sort(full, axis=2))
    t = np.arange(min(L, K))          # rows with at most K valid positions: 0 .. t, then -1
    expect = np.where(np.arange(K)[None, :] <= t[:, None], np.arange(K)[None, :], -1)
    assert np.array_equal(fast[0, :min(L, K)], expect)
    # and the bypassed call's sets against the oracle's, on rows on both sides of k
    rows = np.array(sorted({0, 1, K // 2, K - 2, K - 1, K, K + 1, L - 2, L - 1} & set(range(L))))
    _, _, osc = indexer.prefill(inp, K, rows=rows, want_scores=True)
    check_topk_rows(fast[0][rows], None, osc[0], rows + 1, K, where=f"bypass {dtype} vs oracle")


def test_bypass_in_chunks_against_the_cache():
    q0, Lq, K = 100, 3000, 2048
    L = q0 + Lq
    inp = synth.prefill_inputs(1, L, 64, 128, "fp8", seed=961)
    mpp = (L + 63) // 64
    table = np.random.default_rng(962).permutation(mpp).astype(np.int32)[None, :]
    cache = np.zeros((mpp, 64, 128), np.uint8)
    scales = np.ones((mpp, 64), np.float32)
    s = np.arange(L)
    cache[table[0, s // 64], s % 64] = inp["k"][0]
    scales[table[0, s // 64], s % 64] = inp["k_scale"][0]
    args = [dev(inp["q"][:, q0:]), dev(inp["q_scale"][:, q0:]), dev(inp["w"][:, q0:]), dev(cache), dev(scales),
            dev(table), q0, K]
    fast, _ = dsa.prefill_chunk_paged(*args, want_topk_score=False)
    full, _ = dsa.prefill_chunk_paged(*args, want_topk_score=True)
    torch.cuda.synchronize()
    assert np.array_equal(np.sort(host(fast), axis=2), np.sort(host(full), axis=2))

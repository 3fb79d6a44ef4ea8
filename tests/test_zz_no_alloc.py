"""indexer_prefill_noalloc (the entry point that allocates nothing: its
scratch is a device array inside the library) against indexer_prefill with a
caller workspace, through the C ABI: two calls in a row, the second with a
smaller input, for each fused dtype, and one call that also returns the
score matrix.  The outputs must be the same sets with bit-identical scores
(the two entry points run the same kernels), and sampled rows are checked
against the fp64 oracle as well."""
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


def sorted_rows(idx, val):
    o = np.argsort(idx, axis=-1, kind="stable")
    return np.take_along_axis(idx, o, -1), np.take_along_axis(val, o, -1)


def one_call(dtype, L, H, K, seed, want_scores=False):
    inp = synth.prefill_inputs(1, L, H, 128, dtype, seed=seed)
    args = (dev(inp["q"]), dev(inp["k"]), dev(inp["w"]), K)
    kw = dict(q_scale=dev(inp.get("q_scale")), k_scale=dev(inp.get("k_scale")), want_scores=want_scores)
    say(f"no-alloc prefill {dtype} L={L} H={H} k={K} scores={want_scores}")
    ni, nv, ns = dsa.indexer_prefill_noalloc(*args, **kw)
    torch.cuda.synchronize()
    ri, rv, rs = dsa.indexer_prefill(*args, **kw)
    torch.cuda.synchronize()
    ni, nv, ri, rv = host(ni), host(nv), host(ri), host(rv)
    a_i, a_v = sorted_rows(ni, nv)
    b_i, b_v = sorted_rows(ri, rv)
    assert np.array_equal(a_i, b_i), "index sets differ from indexer_prefill's"
    assert np.array_equal(a_v.view(np.uint32), b_v.view(np.uint32)), "scores differ from indexer_prefill's"
    if want_scores:
        assert np.array_equal(host(ns).view(np.uint32), host(rs).view(np.uint32)), "score matrices differ"
    rows = np.array(sorted({0, 1, K - 1, K, L // 2, L - 1} & set(range(L))))
    _, _, osc = indexer.prefill(inp, K, rows=rows, want_scores=True)
    check_topk_rows(ni[0][rows], nv[0][rows], osc[0], rows + 1, K, where=f"no-alloc {dtype} L={L}")


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_noalloc_two_calls_second_smaller(dtype):
    one_call(dtype, 3000, 64, 256, seed=7100)
    one_call(dtype, 700, 32, 64, seed=7101)


def test_noalloc_with_score_matrix():
    one_call("fp8", 500, 64, 32, seed=7102, want_scores=True)


def test_noalloc_rejects_what_does_not_fit():
    """bf16 at 2 x 65536 keys needs 34 MB of scratch: refused, nothing written."""
    q = torch.zeros((2, 65536, 16, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 65536, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2, 65536, 16), dtype=torch.float32, device="cuda")
    idx = torch.full((2, 65536, 8), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="scratch"):
        dsa.indexer_prefill_noalloc(q, k, w, 8, out=(idx, None, None))
    torch.cuda.synchronize()
    assert bool((idx == 7).all())

"""GPU parity of indexer_prefill_chunk_paged (a chunk of query tokens at
positions q0 .. q0+Lq-1 against the paged fp8 key cache, fp8 or bf16
queries) against the fp64 oracle's prefill rows q0 .. q0+Lq-1 of the whole
sequence, and against the full fused prefill's rows on the GPU (same
per-pair arithmetic: the same selected sets and scores)."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_03_amd as dsa
import synth
from gpu_util import dev, host, run_prefill, say
from oracle import indexer
from oracle.check import check_topk_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def paged_sequence(inp, seed, spare=3):
    """The sequences' fp8 keys placed in a page pool through a permuted table."""
    B, L = inp["k"].shape[:2]
    mpp = (L + 63) // 64
    n_pages = B * mpp + spare
    rng = np.random.default_rng(seed)
    table = rng.permutation(n_pages)[: B * mpp].reshape(B, mpp).astype(np.int32)
    cache = rng.integers(0, 0x7F, size=(n_pages, 64, 128), dtype=np.uint8)   # junk beyond the sequences
    scales = np.ones((n_pages, 64), np.float32)
    s = np.arange(L)
    for b in range(B):
        cache[table[b, s // 64], s % 64] = inp["k"][b]
        scales[table[b, s // 64], s % 64] = inp["k_scale"][b]
    return cache, scales, table


def run_chunk(inp, cache, scales, table, q0, Lq, K):
    q = inp["q"][:, q0:q0 + Lq]
    qs = None if inp.get("q_scale") is None else dev(inp["q_scale"][:, q0:q0 + Lq])
    idx, val = dsa.prefill_chunk_paged(dev(q), qs, dev(inp["w"][:, q0:q0 + Lq]),
                                       dev(cache), dev(scales), dev(table), q0, K)
    torch.cuda.synchronize()
    return host(idx), host(val)


def bf16_queries(inp, seed):
    """The fp8 inputs with their queries replaced by seeded bf16 ones (the
    keys stay fp8: chunks of bf16 queries against the fp8 cache)."""
    rng = np.random.default_rng(seed)
    q = synth.to_bf16_bits(rng.standard_normal(inp["q"].shape, dtype=np.float32))
    return dict(inp, q=q, q_scale=None, q_dtype="bf16")


@pytest.mark.parametrize("qdt", ["fp8", "bf16"])
@pytest.mark.parametrize("B,q0,Lq,H,K", [
    (1, 0, 300, 64, 64),        # the chunk is the whole sequence
    (1, 4000, 100, 64, 2048),   # long rows past 2k: the sampled floor
    (2, 5000, 37, 32, 64),      # ragged chunk, two sequences
    (1, 63, 130, 16, 16),       # chunk start and end off the 64-key pages
    (1, 3000, 200, 48, 256),    # three head blocks (the odd head-sum operand)
])
def test_chunk_matches_oracle_rows(B, q0, Lq, H, K, qdt):
    L = q0 + Lq
    inp = synth.prefill_inputs(B, L, H, 128, "fp8", seed=900 + q0 % 97 + Lq)
    if qdt == "bf16":
        inp = bf16_queries(inp, seed=950 + Lq)
    cache, scales, table = paged_sequence(inp, seed=q0 + Lq)
    say(f"chunk B={B} q0={q0} Lq={Lq} H={H} K={K} queries {qdt}")
    gi, gv = run_chunk(inp, cache, scales, table, q0, Lq, K)
    rows = np.arange(q0, L)
    check_rows = rows if Lq <= 40 else np.concatenate([rows[:8], rows[Lq // 2:Lq // 2 + 4], rows[-8:]])
    _, _, osc = indexer.prefill(inp, K, rows=check_rows, want_scores=True)
    for b in range(B):
        check_topk_rows(gi[b][check_rows - q0], gv[b][check_rows - q0], osc[b], check_rows + 1, K,
                        where=f"chunk b{b}")


def test_chunk_equals_full_prefill_rows():
    q0, Lq, K = 6000, 200, 2048
    L = q0 + Lq
    inp = synth.prefill_inputs(1, L, 64, 128, "fp8", seed=931)
    cache, scales, table = paged_sequence(inp, seed=932)
    say(f"chunk vs full prefill: q0={q0} Lq={Lq}")
    gi, gv = run_chunk(inp, cache, scales, table, q0, Lq, K)
    fi, fv, _ = run_prefill(inp, K)
    a_i, a_v = gi[0], gv[0]
    b_i, b_v = fi[0, q0:], fv[0, q0:]
    oa, ob = np.argsort(a_i, axis=1, kind="stable"), np.argsort(b_i, axis=1, kind="stable")
    assert np.array_equal(np.take_along_axis(a_i, oa, 1), np.take_along_axis(b_i, ob, 1))
    assert np.array_equal(np.take_along_axis(a_v, oa, 1), np.take_along_axis(b_v, ob, 1))


def test_chunk_full_size_sampled():
    # the bench's configuration: the last 4096 tokens of the L=32768 fp8
    # workload against its 32768 keys in a permuted page pool, k=2048
    inp = synth.config_inputs(3)
    L, K = inp["q"].shape[1], 2048
    q0, Lq = L - 4096, 4096
    cache, scales, table = paged_sequence(inp, seed=933, spare=0)
    say(f"chunk full size: q0={q0} Lq={Lq}")
    gi, gv = run_chunk(inp, cache, scales, table, q0, Lq, K)
    rows = np.array([q0, q0 + 1, q0 + 7, q0 + 8, q0 + 2047, q0 + 2048, L - 9, L - 2, L - 1])
    _, _, osc = indexer.prefill(inp, K, rows=rows, want_scores=True)
    check_topk_rows(gi[0][rows - q0], gv[0][rows - q0], osc[0], rows + 1, K, where="chunk full size")
    # every row: k distinct positions inside its history
    assert np.all(gi[0] >= 0) and np.all(gi[0] <= np.arange(q0, L)[:, None])
    srt = np.sort(gi[0], axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])


def ragged_sequence(Lk, q0, Lq, H, seed, qdt="fp8"):
    """One sequence of Lk fp8 keys and, for rows q0 .. q0+Lq-1 only, queries
    (fp8 with scales, or bf16) and softmax weights.  The other query rows
    stay zero (np.zeros: never touched, so a 131072-row query array costs no
    host memory); they are never read.  Draw order: keys, then the chunk's
    queries, then its weight logits."""
    rng = np.random.default_rng(seed)
    kc, ks = synth.quantize_fp8_rows(rng.standard_normal((Lk, 128), dtype=np.float32))
    q = np.zeros((1, Lk, H, 128), np.uint8 if qdt == "fp8" else np.uint16)
    qs = np.ones((1, Lk, H), np.float32) if qdt == "fp8" else None
    w = np.zeros((1, Lk, H), np.float32)
    if Lq:
        src = rng.standard_normal((Lq, H, 128), dtype=np.float32)
        if qdt == "fp8":
            q[0, q0:q0 + Lq], qs[0, q0:q0 + Lq] = synth.quantize_fp8_rows(src)
        else:
            q[0, q0:q0 + Lq] = synth.to_bf16_bits(src)
        w[0, q0:q0 + Lq] = synth.softmax_weights(rng.standard_normal((Lq, H)))
    out = dict(kind="prefill", B=1, L=Lk, H=H, D=128, dtype="fp8", q=q, q_scale=qs, k=kc[None], k_scale=ks[None], w=w)
    if qdt == "bf16":
        out["q_dtype"] = "bf16"
    return out


@pytest.mark.parametrize("K,qdt", [(2048, "fp8"), (64, "fp8"), (2048, "bf16"), (64, "bf16")])
def test_varlen_ragged_batch_against_the_cache(K, qdt):
    """A serving batch of chunks of different lengths at different positions
    in one call: one sequence with no rows, a single-row chunk, chunks off the
    64-key pages, one straddling position 65536 and one ending exactly at
    position 131072 (17-bit positions), all in one permuted page pool.  Every
    row of every chunk against the oracle's row of its own sequence."""
    H = 32
    spec = [(0, 300), (5000, 37), (123, 0), (130900, 172), (65500, 100), (2000, 1)]  # (q0, Lq) per sequence
    seqs = [ragged_sequence(q0 + Lq, q0, Lq, H, seed=970 + i, qdt=qdt) for i, (q0, Lq) in enumerate(spec)]
    B = len(spec)
    pages = [(q0 + Lq + 63) // 64 for q0, Lq in spec]
    mpp = max(pages)
    rng = np.random.default_rng(977)
    pool = rng.permutation(sum(pages) + 5).astype(np.int32)
    table = np.zeros((B, mpp), np.int32)
    cache = rng.integers(0, 0x7F, size=(pool.size, 64, 128), dtype=np.uint8)   # junk outside the sequences
    scales = np.ones((pool.size, 64), np.float32)
    off = 0
    for b, sq in enumerate(seqs):
        table[b, :pages[b]] = pool[off:off + pages[b]]
        off += pages[b]
        s = np.arange(sq["L"])
        cache[table[b, s // 64], s % 64] = sq["k"][0]
        scales[table[b, s // 64], s % 64] = sq["k_scale"][0]
    cu = np.concatenate([[0], np.cumsum([Lq for _, Lq in spec])]).astype(np.int32)
    T = int(cu[-1])
    qpk = np.concatenate([sq["q"][0, q0:q0 + Lq] for sq, (q0, Lq) in zip(seqs, spec)])
    qsp = None if qdt == "bf16" else np.concatenate([sq["q_scale"][0, q0:q0 + Lq] for sq, (q0, Lq) in zip(seqs, spec)])
    wpk = np.concatenate([sq["w"][0, q0:q0 + Lq] for sq, (q0, Lq) in zip(seqs, spec)])
    q_start = np.array([q0 for q0, _ in spec], np.int32)
    say(f"varlen chunk batch: B={B} T={T} K={K} max_kv={max(q0 + Lq for q0, Lq in spec)} queries {qdt}")
    gi, gv = dsa.prefill_chunk_varlen(dev(qpk), None if qsp is None else dev(qsp), dev(wpk), dev(cu), dev(q_start), dev(cache), dev(scales),
                                      dev(table), K, max(q0 + Lq for q0, Lq in spec))
    torch.cuda.synchronize()
    gi, gv = host(gi), host(gv)
    assert gi.shape == (T, K)
    for b, (sq, (q0, Lq)) in enumerate(zip(seqs, spec)):
        if Lq == 0:
            continue
        rows = np.arange(q0, q0 + Lq)
        for a0 in range(0, Lq, 64):
            rr = rows[a0:a0 + 64]
            _, _, osc = indexer.prefill(sq, K, rows=rr, want_scores=True)
            sel = rr - q0 + cu[b]
            check_topk_rows(gi[sel], gv[sel], osc[0], rr + 1, K, where=f"varlen seq {b} (q0={q0})")
        say(f"  sequence {b}: rows {q0}..{q0 + Lq - 1} match the oracle")

"""GPU parity of indexer_decode_paged against the fp64 oracle: scattered and
contiguous page tables, contexts shorter than k, partial last pages, the
full fp8 code range, layout independence (a permuted page table gives
bit-identical results to the identity layout), a sampled candidate floor
that overshoots (full rescoring), and all-tied scores."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_03_amd as dsa
import synth
from gpu_util import dev, host, run_decode, run_prefill, say
from oracle import indexer
from oracle.check import check_topk_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def parity(d, K, name="", queries=None, max_context_len=None):
    B = d["q"].shape[0]
    say(f"decode {name}: B={B} ctx={d['context_lens'][:8].tolist()} H={d['H']} K={K}")
    gi, gv = run_decode(d, K, max_context_len)
    qs = range(B) if queries is None else queries
    swaps = 0
    for b in qs:
        o = indexer.decode_scores(d, b)
        swaps += check_topk_rows(gi[b:b + 1], gv[b:b + 1], o[None], [o.size], K, where=f"{name} q{b}")
    say(f"  ok, near-tie swaps={swaps}")
    return gi, gv


def test_small_scattered_pages():
    d = synth.decode_inputs(5, [100, 64, 130, 30, 1], 64, 128, seed=500, permute=True)
    parity(d, 50, "small")


@pytest.mark.parametrize("H", [16, 32, 48, 64])
def test_head_counts(H):
    d = synth.decode_inputs(3, [5000, 4097, 4095], H, 128, seed=510 + H, permute=True)
    parity(d, 256, f"H={H}")


def test_long_context_k2048():
    d = synth.decode_inputs(4, [20000, 9000, 2048, 2047], 64, 128, seed=520, permute=True)
    gi, _ = parity(d, 2048, "long")
    assert np.all(gi[3, 2047:] == -1) and sorted(gi[3, :2047].tolist()) == list(range(2047))


def test_permuted_equals_identity_bitwise():
    d1 = synth.decode_inputs(3, [3000, 700, 5000], 64, 128, seed=530, permute=True)
    ps = 64
    rows_c, rows_s, bt = [], [], np.zeros_like(d1["block_table"])
    off = 0
    for b in range(3):
        n = -(-int(d1["context_lens"][b]) // ps)
        for j in range(n):
            p = d1["block_table"][b, j]
            rows_c.append(d1["k_cache"][p])
            rows_s.append(d1["k_scale"][p])
            bt[b, j] = off + j
        off += n
    d2 = dict(d1, k_cache=np.stack(rows_c), k_scale=np.stack(rows_s), block_table=bt)
    i1, v1 = run_decode(d1, 300)
    i2, v2 = run_decode(d2, 300)
    for b in range(3):
        o1 = np.argsort(i1[b])
        o2 = np.argsort(i2[b])
        assert np.array_equal(i1[b][o1], i2[b][o2])
        assert np.array_equal(v1[b][o1].view(np.uint32), v2[b][o2].view(np.uint32))


def test_every_fp8_code_decodes():
    """A cache whose 256 tokens hold each E4M3 code (except the two NaNs,
    replaced by 0) in dim 0; the query is +1 on head 0 and -1 on head 1
    in dim 0, so every code's value reaches a score through one ReLU."""
    H, D, K = 16, 128, 2048
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    kc = np.zeros((4, 64, D), np.uint8)
    kc.reshape(256, D)[:, 0] = codes
    ks = np.full((4, 64), 0.5, np.float32)
    q = np.zeros((1, H, D), np.float32)
    q[0, 0, 0], q[0, 1, 0] = 1.0, -1.0
    w = np.zeros((1, H), np.float32)
    w[0, :2] = 1.0
    d = dict(q=synth.to_bf16_bits(q), w=w, k_cache=kc, k_scale=ks,
             block_table=np.arange(4, dtype=np.int32)[None], context_lens=np.array([256], np.int32),
             page_size=64, q_dtype="bf16", H=H)
    parity(d, K, "fp8 codes")


def test_max_context_bound_smaller_than_table():
    d = synth.decode_inputs(2, [500, 300], 64, 128, seed=540, permute=True, max_pages_per_seq=20)
    parity(d, 100, "bound", max_context_len=512)


def test_prefill_row_matches_decode_of_prefix():
    """Row t of an fp8 prefill and a decode with ctx = t+1 over the same keys
    agree within tolerance (the query rows are fp8 values, exactly bf16)."""
    L, H, D, K = 700, 64, 128, 64
    inp = synth.prefill_inputs(1, L, H, D, "fp8", seed=550)
    inp["q_scale"][:] = 1.0   # query values are then fp8 codes, exactly bf16
    gi, gv, gs = run_prefill(inp, K, want_scores=True)
    from oracle import formats
    for t in (63, 64, 699):
        qv = formats.decode(inp["q"][0, t], "fp8", inp["q_scale"][0, t]).astype(np.float32)
        qb = synth.to_bf16_bits(qv)
        assert np.array_equal(synth.gen.bf16_bits_to_f32(qb), qv)  # exact in bf16
        ctx = t + 1
        npg = -(-ctx // 64)
        kc = np.zeros((npg, 64, D), np.uint8)
        ks = np.ones((npg, 64), np.float32)
        kc.reshape(-1, D)[:ctx] = inp["k"][0, :ctx]
        ks.reshape(-1)[:ctx] = inp["k_scale"][0, :ctx]
        d = dict(q=qb[None], w=inp["w"][0, t:t + 1], k_cache=kc, k_scale=ks,
                 block_table=np.arange(npg, dtype=np.int32)[None], context_lens=np.array([ctx], np.int32),
                 page_size=64, q_dtype="bf16", H=H)
        di, dv = run_decode(d, K)
        o = indexer.decode_scores(d, 0)
        check_topk_rows(di, dv, o[None], [ctx], K, where=f"decode t={t}")
        check_topk_rows(gi[0, t:t + 1], gv[0, t:t + 1], gs[0, t:t + 1, :ctx].astype(np.float64), [ctx], K,
                        where=f"prefill-vs-gpu-scores t={t}")


def test_ragged_contexts_with_empty_queries():
    d = synth.decode_inputs(9, [0, 5000, 0, 64, 65, 0, 131, 4096, 1], 64, 128, seed=560, permute=True)
    gi, gv = parity(d, 100, "ragged")
    for b in (0, 2, 5):
        assert np.all(gi[b] == -1) and np.all(np.isneginf(gv[b]))


def test_all_contexts_empty():
    d = synth.decode_inputs(3, [0, 0, 0], 16, 128, seed=561, permute=False, extra_pages=2, max_pages_per_seq=4)
    gi, gv = run_decode(d, 64)
    assert np.all(gi == -1) and np.all(np.isneginf(gv))


def test_many_queries_short_contexts():
    """More queries than waves in the persistent grid have pages: every
    wave share boundary falls inside some query."""
    rng = np.random.default_rng(562)
    ctx = rng.integers(1, 700, size=300).tolist()
    d = synth.decode_inputs(300, ctx, 16, 128, seed=562, permute=True)
    parity(d, 128, "many", queries=range(0, 300, 7))


def sampled_logical_pages(b, ctx, K, page=64, stride=32, max_pages=32):
    """Logical pages the decode scan scores first, to set a query's candidate
    floor: one page in `stride` (sparser when that would exceed `max_pages`
    pages) from a per-query offset (a multiplicative hash of the query index
    scaled to the stride), for queries with ctx >= 4k spanning at least two
    strides of pages."""
    npg = -(-ctx // page)
    stride = max(stride, -(-npg // max_pages))
    if ctx < 4 * K or npg < 2 * stride:
        return []
    off = (((b * 0x9E3779B1) & 0xFFFFFFFF) * stride) >> 32
    return [off + stride * i for i in range((npg - stride) // stride + 1)]


@pytest.mark.parametrize("ctx,K,seed", [([9000, 5000, 300], 512, 570),
                                         # strides 35 and 64: contexts beyond 1024 pages sample sparser
                                         ([70000, 131072, 5000], 2048, 572)])
def test_floor_overshoot_is_repaired(ctx, K, seed):
    """Key scales of the sampled pages raised 50x: the floor taken from the
    sample lies far above each query's k-th largest score, fewer than k
    scores reach it, and the query is rescored in full.  The result still
    matches the oracle, and the query's candidate count (word 1 of its
    counter block in the workspace) equals its context."""
    B = len(ctx)
    d = synth.decode_inputs(B, ctx, 64, 128, seed=seed, permute=True)
    hot = 0
    for b in range(B):
        for j in sampled_logical_pages(b, ctx[b], K):
            d["k_scale"][d["block_table"][b, j]] *= 50.0
            hot += 1
    assert hot > 0
    mcl = max(ctx)
    stride = -(-mcl // 64) * 64
    say(f"decode overshoot: ctx={ctx} K={K} hot pages={hot}")
    ws = torch.zeros(dsa.decode_workspace_bytes(B, mcl, 64, 128, K), dtype=torch.uint8, device="cuda")
    gi, gv = dsa.indexer_decode_paged(dev(d["q"]), dev(d["w"]), dev(d["k_cache"]), dev(d["k_scale"]),
                                      dev(d["block_table"]), dev(d["context_lens"]), K,
                                      max_context_len=mcl, workspace=ws)
    torch.cuda.synchronize()
    gi, gv = host(gi), host(gv)
    for b in range(B):
        o = indexer.decode_scores(d, b)
        check_topk_rows(gi[b:b + 1], gv[b:b + 1], o[None], [o.size], K, where=f"overshoot q{b}")
    ctrl = host(ws[B * stride * 8:B * stride * 8 + B * 64 * 4]).view(np.uint32).reshape(B, 64)
    say(f"  candidate counts {ctrl[:, 1].tolist()}")
    for b in range(B):
        if sampled_logical_pages(b, ctx[b], K):
            assert ctrl[b, 1] == ctx[b]


def test_constant_scores_long_context():
    """Every key zero: all scores tie at 0, the sampled floor admits every
    position, and the ties go to the lowest positions."""
    K = 2048
    d = synth.decode_inputs(2, [20000, 9000], 16, 128, seed=571, permute=True)
    d["k_cache"][:] = 0
    gi, gv = run_decode(d, K)
    for b in range(2):
        assert np.array_equal(np.sort(gi[b]), np.arange(K)), f"q{b}: ties not broken toward low positions"
        assert np.all(gv[b] == 0.0)


@pytest.mark.parametrize("B", [256, 257])
def test_fused_sampling_at_half_grid(B):
    """Sampled queries at H=64 around half the scan's resident grid (two
    workgroups per CU): 256 queries sample inside the scan with every second
    workgroup a sampler, 257 take the separate sample kernel."""
    rng = np.random.default_rng(574 + B)
    ctx = rng.integers(4096, 6000, size=B).tolist()
    d = synth.decode_inputs(B, ctx, 64, 128, seed=574 + B, permute=True)
    parity(d, 256, f"B={B} sampled", queries=list(range(0, B, 4)) + [B - 1])


def test_batch_beyond_fused_sampling():
    """300 sampled queries at H=64: more than half the scan's resident grid,
    so the sample runs as a kernel of its own before the scan."""
    rng = np.random.default_rng(573)
    ctx = rng.integers(5000, 12000, size=300).tolist()
    d = synth.decode_inputs(300, ctx, 64, 128, seed=573, permute=True)
    parity(d, 512, "B=300 sampled", queries=list(range(0, 300, 5)) + [299])


def test_batch_beyond_lds_prefix():
    """2100 queries: the scan's page prefix over queries no longer fits its
    LDS table and comes from global memory instead."""
    rng = np.random.default_rng(572)
    ctx = rng.integers(1, 300, size=2100).tolist()
    d = synth.decode_inputs(2100, ctx, 16, 128, seed=572, permute=True)
    parity(d, 64, "B=2100", queries=list(range(0, 2100, 97)) + [2099])


def test_workspace_garbage_then_reused():
    """The caller's workspace starts as 0xFF bytes (every counter word at its
    maximum, every floor word marked as published), and is then reused
    unchanged by a second call with another batch: each query's counters are
    cleared by the call itself, so both results match the oracle."""
    K = 512
    d1 = synth.decode_inputs(4, [20000, 9000, 4096, 700], 64, 128, seed=575, permute=True)
    rng = np.random.default_rng(576)
    ctx2 = rng.integers(4096, 9000, size=300).tolist()
    d2 = synth.decode_inputs(300, ctx2, 64, 128, seed=576, permute=True)
    # each call's counter blocks sit after its own candidate lists, so the
    # second call's lie over the first call's candidates
    mcl = {id(d): d["block_table"].shape[1] * 64 for d in (d1, d2)}
    nws = max(dsa.decode_workspace_bytes(d["q"].shape[0], mcl[id(d)], 64, 128, K) for d in (d1, d2))
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    for d, name, qs in ((d1, "garbage workspace", range(4)),
                        (d2, "reused workspace, B=300", list(range(0, 300, 6)) + [299]),
                        (d1, "reused again, B=4", range(4))):
        say(f"decode {name}: B={d['q'].shape[0]} K={K}")
        gi, gv = dsa.indexer_decode_paged(dev(d["q"]), dev(d["w"]), dev(d["k_cache"]), dev(d["k_scale"]),
                                          dev(d["block_table"]), dev(d["context_lens"]), K,
                                          max_context_len=mcl[id(d)], workspace=ws)
        torch.cuda.synchronize()
        gi, gv = host(gi), host(gv)
        for b in qs:
            o = indexer.decode_scores(d, b)
            check_topk_rows(gi[b:b + 1], gv[b:b + 1], o[None], [o.size], K, where=f"{name} q{b}")
        say("  ok")

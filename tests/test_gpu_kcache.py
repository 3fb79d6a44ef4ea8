"""GPU parity of indexer_kcache_append (per-token FP8 quantisation and paged
append) against the oracle (oracle/kcache.py): bit-exact codes and scales
over the whole cache, untouched slots left as they were, exact midpoints,
signed zeros, all-zero keys, saturation, the skip rules, and a cache
written by the kernel then read by the paged decode."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_03_amd as dsa
import synth
from gpu_util import dev, host, run_decode, say
from oracle import indexer
from oracle.check import check_topk_rows
from oracle.kcache import kcache_append as oracle_append

pytestmark = pytest.mark.gpu

SENTINEL_CODE, SENTINEL_SCALE = 0x11, -1.0


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_append(cache, scales, keys, dtype, seq, pos, table):
    k = torch.from_numpy(np.ascontiguousarray(keys).view(np.int16)).cuda() if dtype == "bf16" else dev(keys)
    kc, ks = dev(cache), dev(scales)
    dsa.kcache_append(k, dev(seq.astype(np.int32)), dev(pos.astype(np.int32)), dev(table.astype(np.int32)),
                      kc, ks)
    torch.cuda.synchronize()
    return host(kc), host(ks)


def check_exact(name, cache, scales, keys, dtype, seq, pos, table):
    say(f"kcache {name}: T={len(seq)} dtype={dtype} pages={cache.shape[0]}")
    g_cache, g_scales = run_append(cache, scales, keys, dtype, seq, pos, table)
    o_cache, o_scales = oracle_append(cache, scales, keys, dtype, seq, pos, table)
    bad = np.argwhere(g_cache != o_cache)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}: " \
                          f"gpu {g_cache[tuple(bad[0])]:#x} oracle {o_cache[tuple(bad[0])]:#x}"
    assert np.array_equal(g_scales.view(np.uint32), o_scales.view(np.uint32)), "scales differ"
    return g_cache, g_scales


def random_layout(rng, B, pages_per_seq, n_pages):
    perm = rng.permutation(n_pages)[: B * pages_per_seq]
    return perm.reshape(B, pages_per_seq).astype(np.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_random_keys_scattered_pages(dtype):
    rng = np.random.default_rng(21)
    B, mpp, n_pages, D = 3, 8, 40, 128
    table = random_layout(rng, B, mpp, n_pages)
    T = 1001  # ragged against the kernel's four keys per lane group
    seq = rng.integers(0, B, T)
    pos = np.empty(T, np.int64)
    for b in range(B):  # distinct positions within each sequence
        m = seq == b
        pos[m] = rng.permutation(mpp * 64)[: m.sum()]
    x = rng.normal(size=(T, D)) * np.exp(rng.uniform(-4, 4, size=(T, 1)))
    keys = synth.to_bf16_bits(x.astype(np.float32)) if dtype == "bf16" else x.astype(np.float32)
    cache = np.full((n_pages, 64, D), SENTINEL_CODE, np.uint8)
    scales = np.full((n_pages, 64), SENTINEL_SCALE, np.float32)
    check_exact("random", cache, scales, keys, dtype, seq, pos, table)


def test_midpoints_signed_zeros_and_saturation():
    D = 128
    rows = []
    # scale exactly 1 (absmax 448): the quotient is the value itself
    r = np.zeros(D, np.float32)
    r[0] = 448.0
    mids = [1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 432.0, -1.0625, -432.0, 0.0, -0.0, 2.0 ** -12,
            -(2.0 ** -12), 0.875 * 2.0 ** -6, 15.5, 17.0, -240.0, 1.0]
    r[1:1 + len(mids)] = mids
    rows.append(r)
    rows.append(np.zeros(D, np.float32))                         # all zero: scale 1, codes 0
    z = np.zeros(D, np.float32)
    z[::2] = -0.0
    rows.append(z)                                               # signed zeros
    rows.append(np.full(D, -896.0, np.float32))                  # scale 2, all -448
    s = np.linspace(-1.0, 1.0, D).astype(np.float32) * np.float32(3.0e-30)  # tiny magnitudes
    rows.append(s)
    t = np.linspace(-1.0, 1.0, D).astype(np.float32) * np.float32(2.0e30)   # huge magnitudes
    rows.append(t)
    keys = np.stack(rows)
    T = len(rows)
    table = np.arange(4, dtype=np.int32)[None, :]
    cache = np.full((4, 64, D), SENTINEL_CODE, np.uint8)
    scales = np.full((4, 64), SENTINEL_SCALE, np.float32)
    g, gs = check_exact("midpoints", cache, scales, keys, "f32", np.zeros(T), np.arange(T) * 37, table)
    assert list(g[0, 0, 1:9]) == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0xB8, 0xFE, 0x00]
    assert g[0, 0, 9] == 0x80 and gs[0, 37] == 1.0 and not g[0, 37].any()


def test_skip_rules_leave_slots_untouched():
    rng = np.random.default_rng(5)
    B, mpp, n_pages, D = 2, 3, 8, 128
    table = random_layout(rng, B, mpp, n_pages)
    seq = np.array([0, 1, -1, 2, 0, 1, 0, 1, -7])
    pos = np.array([0, 191, 5, 5, 192, -1, 100, 64, 3])   # keys 2, 3, 4, 5 and 8 are skipped
    keys = rng.normal(size=(len(seq), D)).astype(np.float32)
    cache = np.full((n_pages, 64, D), SENTINEL_CODE, np.uint8)
    scales = np.full((n_pages, 64), SENTINEL_SCALE, np.float32)
    g, gs = check_exact("skips", cache, scales, keys, "f32", seq, pos, table)
    assert int((gs != SENTINEL_SCALE).sum()) == 4


def test_large_append_then_decode_reads_it():
    # one 131072-token context written by the kernel, then scored by the paged decode
    rng = np.random.default_rng(9)
    D, H, K, ctx = 128, 64, 2048, 131072
    n_pages = ctx // 64
    table = rng.permutation(n_pages).astype(np.int32)[None, :]
    keys = synth.to_bf16_bits(rng.normal(size=(ctx, D)).astype(np.float32))
    cache = np.zeros((n_pages, 64, D), np.uint8)
    scales = np.zeros((n_pages, 64), np.float32)
    g_cache, g_scales = check_exact("large", cache, scales, keys, "bf16", np.zeros(ctx), rng.permutation(ctx),
                                    table)
    q = synth.to_bf16_bits(rng.normal(size=(1, H, D)).astype(np.float32))
    w = synth.softmax_weights(rng.normal(size=(1, H))).astype(np.float32)
    d = dict(q=q, w=w, k_cache=g_cache, k_scale=g_scales, block_table=table,
             context_lens=np.array([ctx], np.int32), H=H, page_size=64)
    gi, gv = run_decode(d, K)
    o = indexer.decode_scores(d, 0)
    check_topk_rows(gi, gv, o[None], [ctx], K, where="decode of the appended cache")


def test_full_size_bulk_append_sampled():
    # the bench's configuration: 64 sequences x 131072 bf16 keys (seeded on the
    # device), identity block table; sampled keys checked bit for bit
    dev = torch.device("cuda")
    B, ctx = 64, 131072
    T = B * ctx
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    kn = torch.randn((T, 128), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ar = torch.arange(T, device=dev, dtype=torch.int32)
    table = torch.arange(B * ctx // 64, device=dev, dtype=torch.int32).reshape(B, ctx // 64)
    cache = torch.zeros((B * ctx // 64, 64, 128), dtype=torch.uint8, device=dev)
    scale = torch.zeros((B * ctx // 64, 64), dtype=torch.float32, device=dev)
    say(f"kcache full size: T={T}")
    dsa.kcache_append(kn, ar // ctx, ar % ctx, table, cache, scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    pick = np.concatenate([[0, T - 1, ctx - 1, ctx], rng.integers(0, T, 4000)])
    keys = kn[torch.from_numpy(pick).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    from oracle.kcache import key_rows_to_f32, quantize_keys
    codes, sc = quantize_keys(key_rows_to_f32(keys, "bf16"))
    rows = torch.from_numpy(pick).to(dev)  # identity table: key i sits in row i of the flattened pool
    g_codes = cache.view(-1, 128)[rows].cpu().numpy()
    g_sc = scale.view(-1)[rows].cpu().numpy()
    assert np.array_equal(g_codes, codes)
    assert np.array_equal(g_sc.view(np.uint32), sc.view(np.uint32))
    # every slot was written (no zero scale left)
    assert bool((scale > 0).all())


def test_decode_step_append_score_gather():
    # one serving step for 3 sequences: append each new token's key at its
    # position, score the query over its whole context (the new key included),
    # then gather the selected rows of a latent cache with the same paging
    from oracle.gather import topk_gather as oracle_gather
    d = synth.decode_inputs(3, [3000, 700, 4500], 64, 128, seed=71, permute=True)
    ctx = d["context_lens"].astype(np.int64)
    rng = np.random.default_rng(72)
    new = synth.to_bf16_bits(rng.normal(size=(3, 128)).astype(np.float32))
    pos = (ctx - 1).astype(np.int32)   # each query's own position: its key enters before scoring
    seq = np.arange(3, dtype=np.int32)
    kc, ks = dev(d["k_cache"]), dev(d["k_scale"])
    k_new = torch.from_numpy(new.view(np.int16)).cuda()
    dsa.kcache_append(k_new, dev(seq), dev(pos), dev(d["block_table"]), kc, ks)
    torch.cuda.synchronize()
    o_cache, o_scales = oracle_append(d["k_cache"], d["k_scale"], new, "bf16", seq, pos, d["block_table"])
    assert np.array_equal(host(kc), o_cache) and np.array_equal(host(ks).view(np.uint32), o_scales.view(np.uint32))
    d2 = dict(d, k_cache=o_cache, k_scale=o_scales)
    K = 256
    gi, gv = dsa.indexer_decode_paged(dev(d["q"]), dev(d["w"]), kc, ks, dev(d["block_table"]),
                                      dev(d["context_lens"]), K)
    torch.cuda.synchronize()
    gi, gv = host(gi), host(gv)
    for b in range(3):
        o = indexer.decode_scores(d2, b)
        check_topk_rows(gi[b:b + 1], gv[b:b + 1], o[None], [o.size], K, where=f"step q{b}")
    latent = rng.integers(0, 256, size=(d["k_cache"].shape[0], 64, 1024), dtype=np.uint8)
    rows = host(dsa.topk_gather(dev(latent), dev(d["block_table"]), dev(gi)))
    assert np.array_equal(rows, oracle_gather(latent, d["block_table"], gi))

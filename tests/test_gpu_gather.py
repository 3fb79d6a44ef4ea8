"""GPU parity of indexer_topk_gather (rows of a paged latent cache at the
selected positions) against the oracle (oracle/gather.py): exact bytes, with
padding and out-of-table indices, several row sizes and ragged B * K, the
paged decode's own output as the indices, and the full-size configuration
the bench times (sampled rows).  Also Index Share's multi-layer gather
(indexer_topk_gather_layers): every layer's output against the oracle's
gather of that layer, from 2 to 64 layers in one launch."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_03_amd as dsa
import synth
from gpu_util import dev, host, run_decode, say
from oracle.gather import topk_gather as oracle_gather
from oracle.gather import topk_gather_layers as oracle_gather_layers

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("B,K,row", [(3, 7, 1024), (4, 100, 16), (2, 33, 48), (5, 64, 4096), (1, 9, 65536)])
def test_random_indices(B, K, row):
    rng = np.random.default_rng(B * 1000 + K + row)
    mpp, n_pages = 6, B * 6 + 3
    say(f"gather B={B} K={K} row={row}")
    cache = rng.integers(0, 256, size=(n_pages, 64, row), dtype=np.uint8)
    table = rng.permutation(n_pages)[: B * mpp].reshape(B, mpp).astype(np.int32)
    idx = rng.integers(0, mpp * 64, size=(B, K)).astype(np.int32)
    idx[rng.random((B, K)) < 0.1] = -1                         # padding
    idx[0, 0] = mpp * 64                                       # past the table
    idx[-1, -1] = -5
    out = host(dsa.topk_gather(dev(cache), dev(table), dev(idx)))
    assert np.array_equal(out, oracle_gather(cache, table, idx))


def test_decode_output_feeds_the_gather():
    d = synth.decode_inputs(3, [5000, 700, 130], 64, 128, seed=61, permute=True)
    gi, _ = run_decode(d, 512)
    rng = np.random.default_rng(62)
    n_pages = d["k_cache"].shape[0]
    latent = synth.to_bf16_bits(rng.normal(size=(n_pages, 64, 512)).astype(np.float32))   # d_c = 512, bf16
    out = dsa.topk_gather(dev(latent), dev(d["block_table"]), dev(gi))
    torch.cuda.synchronize()
    got = host(out).view(np.uint16)
    ref = oracle_gather(latent.view(np.uint8).reshape(n_pages, 64, 1024), d["block_table"], gi).view(np.uint16)
    assert np.array_equal(got, ref.reshape(got.shape))
    assert np.all(got[2, 130:] == 0)  # the short query's padding rows are zero


def test_full_size_sampled():
    # the bench's configuration: 64 queries x 2048 selected positions from
    # 131072-token contexts of 1024-byte rows (512 bf16), identity layout
    B, K, ctx, row = 64, 2048, 131072, 1024
    n_pages = B * ctx // 64
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    say(f"gather full size: {n_pages * 64 * row / 1e9:.1f} GB latent cache")
    cache = torch.randint(0, 256, (n_pages, 64, row), generator=g, device="cuda", dtype=torch.uint8)
    table = torch.arange(n_pages, device="cuda", dtype=torch.int32).reshape(B, ctx // 64)
    idx = torch.randint(0, ctx, (B, K), generator=g, device="cuda", dtype=torch.int32)
    idx[:, -3:] = -1
    out = dsa.topk_gather(cache, table, idx)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    bs = rng.integers(0, B, 3000)
    js = np.concatenate([[0, K - 4, K - 1], rng.integers(0, K, 2997)])
    h_idx = host(idx)
    s = h_idx[bs, js]
    flat = cache.view(-1, row)
    rows = torch.from_numpy((bs.astype(np.int64) * ctx + np.maximum(s, 0))).cuda()
    expect = host(flat[rows]) * (s >= 0)[:, None].astype(np.uint8)
    got = host(out[torch.from_numpy(bs).cuda(), torch.from_numpy(js).cuda()])
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("S,B,K,row", [(3, 5, 300, 656), (61, 1, 64, 1152), (64, 2, 33, 48), (2, 16, 2048, 1024)])
def test_layers_share_one_selection(S, B, K, row):
    """Index Share: S layers gather the same selection from their own caches
    in one launch (one grid row per layer), from a 16-wave selection over 61
    layers to an 8192-wave one over 2."""
    rng = np.random.default_rng(S * 7919 + B * 131 + K + row)
    mpp, n_pages = 5, B * 5 + 2
    say(f"gather layers S={S} B={B} K={K} row={row}")
    caches = [rng.integers(0, 256, size=(n_pages, 64, row), dtype=np.uint8) for _ in range(S)]
    table = rng.permutation(n_pages)[: B * mpp].reshape(B, mpp).astype(np.int32)
    idx = rng.integers(0, mpp * 64, size=(B, K)).astype(np.int32)
    idx[rng.random((B, K)) < 0.1] = -1
    idx[0, 0] = mpp * 64
    outs = dsa.topk_gather_layers([dev(c) for c in caches], dev(table), dev(idx))
    torch.cuda.synchronize()
    want = oracle_gather_layers(caches, table, idx)
    for l in range(S):
        assert np.array_equal(host(outs[l]), want[l]), f"layer {l}"


def test_layers_match_the_single_layer_gather():
    """The multi-layer launch writes, per layer, exactly what a single-layer
    gather writes (decode output as indices, bf16 latent rows)."""
    d = synth.decode_inputs(2, [3000, 200], 64, 128, seed=63, permute=True)
    gi, _ = run_decode(d, 256)
    rng = np.random.default_rng(64)
    n_pages = d["k_cache"].shape[0]
    lat = [dev(synth.to_bf16_bits(rng.normal(size=(n_pages, 64, 512)).astype(np.float32))) for _ in range(4)]
    bt, ix = dev(d["block_table"]), dev(gi)
    outs = dsa.topk_gather_layers(lat, bt, ix)
    for l in range(4):
        assert torch.equal(outs[l], dsa.topk_gather(lat[l], bt, ix)), f"layer {l}"

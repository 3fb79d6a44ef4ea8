"""GPU parity of indexer_prefill against the fp64 oracle: the tiny fp32
workload with its full score matrix, edge lengths on both the generic and
the fused MFMA paths, the hand-worked example, tie-heavy keys and small k
(many buffer compactions)."""
import json
import os

import numpy as np
import pytest
import torch

import synth
from gpu_util import run_prefill, say
from oracle import indexer
from oracle.check import check_scores, check_topk_rows

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand8.json")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def parity(inp, K, want_scores=False, rows=None, name=""):
    B, L = inp["q"].shape[:2]
    say(f"prefill {name}: dtype={inp['dtype']} B={B} L={L} H={inp['q'].shape[2]} D={inp['q'].shape[3]} K={K}")
    gi, gv, gs = run_prefill(inp, K, want_scores)
    rows = np.arange(L) if rows is None else np.asarray(rows)
    oi, ov, osc = indexer.prefill(inp, K, rows=rows, want_scores=True)
    mag = None
    if np.any(np.asarray(inp["w"]) < 0):  # signed weights: tolerances scale with the magnitude sums
        _, _, mag = indexer.prefill(dict(inp, w=np.abs(inp["w"])), K, rows=rows, want_scores=True)
    swaps = 0
    for b in range(B):
        mb = None if mag is None else mag[b]
        if want_scores:
            check_scores(gs[b][rows], osc[b], what=f"{name} scores b={b}", mag=mb)
        swaps += check_topk_rows(gi[b][rows], gv[b][rows], osc[b], rows + 1, K, where=f"{name} b={b}", mag=mb)
    say(f"  ok, near-tie swaps={swaps}")
    return gi, gv


def test_tiny_fp32_workload_full_matrix():
    """Workload 1: L=256, H=4, D=32, k=16, fp32; rows t < 15 are padded."""
    inp = synth.config_inputs(1)
    gi, _ = parity(inp, 16, want_scores=True, name="tiny")
    assert np.all(gi[0, :15, -1] == -1) and np.all(gi[0, 15:] >= 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 63, 64, 65, 300])
def test_generic_path_edge_lengths(dtype, L):
    inp = synth.prefill_inputs(1, L, 8, 32, dtype, seed=1000 + L)
    parity(inp, 16, want_scores=True, name=f"generic L={L}")


@pytest.mark.parametrize("dtype,D,H,L,K", [("f32", 128, 64, 200, 16), ("f32", 64, 60, 130, 32),
                                           ("bf16", 128, 20, 257, 64), ("bf16", 32, 64, 100, 8),
                                           ("fp8", 128, 36, 190, 48), ("fp8", 64, 12, 129, 128)])
def test_generic_path_shapes(dtype, D, H, L, K):
    """Shapes outside the fused kernels (fp32 inputs, D below 128, H not a
    multiple of 16) at the ends of the supported ranges: every D, H up to 64,
    several key tiles with a ragged last one, k above some rows' lengths."""
    inp = synth.prefill_inputs(1, L, H, D, dtype, seed=1100 + D + H + L)
    parity(inp, K, want_scores=True, name=f"generic D={D} H={H}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("L,H,K", [(1, 64, 16), (17, 64, 16), (64, 16, 16), (65, 64, 64), (1000, 64, 64),
                                   (1000, 32, 7), (5000, 16, 2048), (300, 48, 32), (3000, 48, 256)])
def test_fused_path(dtype, L, H, K):
    inp = synth.prefill_inputs(1, L, H, 128, dtype, seed=2000 + L + H)
    parity(inp, K, want_scores=(L <= 1000), name=f"fused L={L} H={H}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_fused_batch2_and_generic_d64(dtype):
    inp = synth.prefill_inputs(2, 200, 16, 128, dtype, seed=3000)
    parity(inp, 32, want_scores=True, name="fused B=2")
    inp = synth.prefill_inputs(2, 130, 12, 64, dtype, seed=3001)
    parity(inp, 32, want_scores=True, name="generic D=64 B=2")


def hand_inputs(dtype, D, H=16):
    """The hand-worked 8-token example embedded in H heads of width D (extra
    heads get weight 0, extra dims are 0)."""
    g = json.load(open(GOLD))
    q = np.zeros((1, 8, H, D), np.float32)
    k = np.zeros((1, 8, D), np.float32)
    q[0, :, :2, :4] = np.array(g["q_heads"], np.float32)[None]
    k[0, :, :4] = np.array(g["k"], np.float32)
    w = np.zeros((1, 8, H), np.float32)
    w[..., :2] = np.array(g["w"], np.float32)
    inp = dict(q=q, k=k, w=w, dtype="f32", q_scale=None, k_scale=None)
    if dtype == "bf16":
        inp.update(q=synth.to_bf16_bits(q), k=synth.to_bf16_bits(k), dtype="bf16")
    elif dtype == "fp8":
        inp.update(q=torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy(),
                   k=torch.from_numpy(k).to(torch.float8_e4m3fn).view(torch.uint8).numpy(),
                   q_scale=np.ones(q.shape[:3], np.float32), k_scale=np.ones(k.shape[:2], np.float32),
                   dtype="fp8")
    return g, inp


@pytest.mark.parametrize("dtype,D,H", [("f32", 64, 4), ("bf16", 64, 4), ("fp8", 64, 4),
                                       ("bf16", 128, 16), ("fp8", 128, 16)])
def test_hand_worked_example(dtype, D, H):
    g, inp = hand_inputs(dtype, D, H)
    gi, gv, gs = run_prefill(inp, 3, want_scores=True)
    exp = np.array(g["scores"]) / np.sqrt(D / 4.0)
    if D == 64:   # 1/sqrt(64) = 1/8 keeps every value exact: bit-exact match
        assert np.array_equal(gs[0, 7], exp.astype(np.float32))
    else:
        check_scores(gs[0, 7], exp)
    for t in range(8):
        assert sorted(x for x in gi[0, t].tolist() if x >= 0) == g["topk3_sets"][t], t


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_tie_heavy_keys_fused(dtype):
    inp = synth.tie_heavy_prefill(1, 3000, 64, 128, dtype, seed=4000, n_proto=4)
    gi, gv = parity(inp, 256, name="ties fused")
    # identical keys give bit-identical scores: among the GPU's own equal
    # scores the lower positions must be the ones kept
    _, _, sc = run_prefill(inp, 256, want_scores=True)
    for t in (2999, 2500, 1024):
        row = sc[0, t, : t + 1]
        sel = set(gi[0, t].tolist())
        kth = np.sort(gv[0, t])[0]
        eq = np.flatnonzero(row == kth)
        taken = [s for s in eq if s in sel]
        assert taken == sorted(eq.tolist())[: len(taken)]


def test_tie_heavy_generic():
    inp = synth.tie_heavy_prefill(1, 500, 4, 32, "f32", seed=4001, n_proto=3)
    parity(inp, 40, want_scores=True, name="ties generic")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_fused_small_k_long_rows_sampled(dtype):
    """Long rows with a small k: the staged kernels' candidate buffers are cut
    down many times per row, under a floor set from a strided sample of
    chunks."""
    L, K = 8192, 64
    inp = synth.prefill_inputs(1, L, 16, 128, dtype, seed=5500)
    rows = np.array([0, 63, 64, 2047, 2048, 4095, 5000, 8190, 8191])
    parity(inp, K, rows=rows, name="small k long rows")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_fused_floor_rescan_when_sample_holds_the_top(dtype):
    """Keys at positions 1024 j + [960, 1024) -- the strided chunks a long row
    of the staged kernels scores first -- score far above every other key, so
    the floor each long row sets from that sample lies above its k-th score:
    the check at the end of the scan fails and the row is scanned again.  The
    selection must still be exact."""
    L, H, D, K = 4096, 16, 128, 256
    rng = np.random.default_rng(6000)
    q0 = rng.standard_normal(D).astype(np.float32)
    q = np.broadcast_to(q0, (1, L, H, D)).copy()
    k = rng.standard_normal((1, L, D)).astype(np.float32)
    hot = (np.arange(L) // 64) % 16 == 15
    k[0, hot] = 2.0 * q0[None, :] + 0.1 * rng.standard_normal((int(hot.sum()), D)).astype(np.float32)
    w = synth.softmax_weights(rng.standard_normal((1, L, H)))
    if dtype == "fp8":
        qc, qs = synth.quantize_fp8_rows(q)
        kc, ks = synth.quantize_fp8_rows(k)
        inp = dict(q=qc, q_scale=qs, k=kc, k_scale=ks, w=w, dtype="fp8")
    else:
        inp = dict(q=synth.to_bf16_bits(q), q_scale=None, k=synth.to_bf16_bits(k), k_scale=None, w=w,
                   dtype="bf16")
    rows = np.array([0, 255, 256, 1983, 1984, 2047, 2048, 3000, 4094, 4095])
    gi, _ = parity(inp, K, rows=rows, name=f"floor rescan {dtype}")
    hot_pos = np.flatnonzero(hot)
    assert set(gi[0, 4095].tolist()) == set(hot_pos.tolist())


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_speculative_cut_rescan_when_early_keys_win(dtype):
    """Key scores fall with position, so a long row's earliest keys are its
    top k.  The sampled floor (strided chunks) is representative, but the
    sequential scan then meets the best keys first: the buffer fills, and
    the speculative cut -- sized for a row whose scanned keys hold k n_seen /
    (t+1) of its top k -- drops some of them.  Fewer than k keys end above
    the floor, the row is scanned again without speculation, and the
    selection must still be exact."""
    L, H, D, K = 8192, 16, 128, 2048
    rng = np.random.default_rng(6100)
    q0 = rng.standard_normal(D).astype(np.float32)
    q = np.broadcast_to(q0, (1, L, H, D)).copy()
    a = 2.0 * (1.0 - np.arange(L, dtype=np.float32) / L)
    k = a[None, :, None] * q0[None, None, :] + 0.3 * rng.standard_normal((1, L, D)).astype(np.float32)
    w = synth.softmax_weights(rng.standard_normal((1, L, H)))
    if dtype == "fp8":
        qc, qs = synth.quantize_fp8_rows(q)
        kc, ks = synth.quantize_fp8_rows(k)
        inp = dict(q=qc, q_scale=qs, k=kc, k_scale=ks, w=w, dtype="fp8")
    else:
        inp = dict(q=synth.to_bf16_bits(q), q_scale=None, k=synth.to_bf16_bits(k), k_scale=None, w=w,
                   dtype="bf16")
    rows = np.array([0, 2047, 2048, 4095, 4096, 6000, 7000, 8190, 8191])
    parity(inp, K, rows=rows, name=f"early keys win {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_tie_heavy_long_rows_sampled(dtype):
    """Exact ties on long rows: ties at the k-th score go to the lowest
    positions even though the fp8 kernel scores a row's chunks out of order."""
    inp = synth.tie_heavy_prefill(1, 6000, 16, 128, dtype, seed=4100, n_proto=4)
    rows = np.array([0, 511, 512, 2100, 4000, 5999])
    parity(inp, 512, rows=rows, name="ties long rows")


@pytest.mark.parametrize("dtype,L", [("fp8", 65536), ("fp8", 66000), ("fp8", 131072),
                                     ("bf16", 65536), ("bf16", 66000), ("bf16", 131072)])
def test_fused_long_sequences_sampled(dtype, L):
    """Both candidate encodings (16-bit positions up to L = 65536, the 17-bit
    encoding beyond, up to the largest supported L), checked on sampled rows
    including the first and last."""
    inp = synth.prefill_inputs(1, L, 16, 128, dtype, seed=5000 + L)
    rows = np.array(sorted(r for r in {0, 2046, 2047, 2048, 40000, 65535, 65536, 100000, L - 2, L - 1} if r < L))
    say(f"prefill long {dtype} L={L}")
    gi, gv, _ = run_prefill(inp, 2048)
    _, _, osc = indexer.prefill(inp, 2048, rows=rows, want_scores=True)
    check_topk_rows(gi[0][rows], gv[0][rows], osc[0], rows + 1, 2048, where=f"long {dtype} L={L}")


def _e4m3(x):
    """float32 array -> E4M3FN codes (saturating RNE), no scaling."""
    t = torch.clamp(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)), -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _finite_e4m3_codes():
    """The 254 E4M3FN codes that are not NaN (0x7F and 0xFF are)."""
    return np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)


@pytest.mark.parametrize("H", [16, 48])
def test_fused_fp8_every_code(H):
    """Every finite E4M3FN code, positive and negative, subnormal and
    saturated, appears in the keys and in the queries of the fused fp8 path
    (unit scales): each code is read by the scaled MFMA both as an A and as a
    B operand, and the scores and selections match the oracle's decoding of
    the same bytes."""
    codes = _finite_e4m3_codes()
    rng = np.random.default_rng(590 + H)
    L, D, K = 260, 128, 32
    k = np.empty((1, L, D), np.uint8)
    q = np.empty((1, L, H, D), np.uint8)
    # keys 0 and 1 hold all 254 codes (then two zeros); the others a permutation each
    k[0, :2] = np.concatenate([codes, np.zeros(2, np.uint8)]).reshape(2, D)
    for s_ in range(2, L):
        k[0, s_] = rng.permutation(codes)[:D]
    # every token's first two heads hold all codes too; the other heads a random draw
    q[0, :, :2] = np.concatenate([codes, np.zeros(2, np.uint8)]).reshape(2, D)[None]
    q[0, :, 2:] = rng.choice(codes, size=(L, H - 2, D))
    inp = dict(kind="prefill", B=1, L=L, H=H, D=D, dtype="fp8", q=q, k=k,
               q_scale=np.ones((1, L, H), np.float32), k_scale=np.ones((1, L), np.float32),
               w=synth.softmax_weights(rng.standard_normal((1, L, H))))
    parity(inp, K, want_scores=True, name=f"fp8 every code H={H}")


@pytest.mark.parametrize("signed", [False, True])
def test_fused_fp8_heads_far_apart(signed):
    """Query heads of one token whose fp8 codes lie 2^0 .. 2^-12 below the
    token's largest head, with head weights that grow as the head shrinks, so
    the small heads carry as much of each score as the large ones: each
    head's ReLU'd dot product must keep its own relative precision (one
    exponent per head, not per token).  Scores are far above the absolute
    floor of the tolerance, so the relative bound decides."""
    rng = np.random.default_rng(583)
    L, H, D, K = 600, 64, 128, 64
    j = rng.integers(0, 13, size=(1, L, H, 1))
    qv = rng.standard_normal((1, L, H, D)).astype(np.float32) * 100.0 * np.exp2(-j)
    kv = rng.standard_normal((1, L, D)).astype(np.float32) * 100.0
    kv[:, ::41] = 0.0
    w = (np.exp2(j[..., 0]) * rng.uniform(0.5, 1.0, size=(1, L, H))).astype(np.float32)
    if signed:
        w *= np.where(rng.random((1, L, H)) < 0.5, -1.0, 1.0).astype(np.float32)
    inp = dict(kind="prefill", B=1, L=L, H=H, D=D, dtype="fp8", q=_e4m3(qv), k=_e4m3(kv),
               q_scale=rng.uniform(0.5, 2.0, size=(1, L, H)).astype(np.float32),
               k_scale=rng.uniform(0.5, 2.0, size=(1, L)).astype(np.float32), w=w)
    parity(inp, K, want_scores=True, name=f"fp8 heads far apart signed={signed}")


@pytest.mark.parametrize("signed", [False, True])
def test_fused_fp8_codes_far_from_full_range(signed):
    """fp8 codes that use little of the E4M3 range (magnitudes spread over
    2^-7 .. 1 per query head and 2^-11 .. 1 per key, arbitrary positive
    scales) and some all-zero keys: every per-token and per-key operand
    scale the fused kernel derives is exercised, and the scores and
    selections match the oracle -- with non-negative head weights under the
    plain tolerance, with signed ones under the magnitude-sum tolerance."""
    rng = np.random.default_rng(580)
    L, H, D, K = 700, 64, 128, 64
    qv = rng.standard_normal((1, L, H, D)).astype(np.float32) * np.exp2(-rng.integers(0, 8, size=(1, L, H, 1)))
    kv = rng.standard_normal((1, L, D)).astype(np.float32) * np.exp2(-rng.integers(0, 12, size=(1, L, 1)))
    kv[:, ::53] = 0.0
    inp = dict(kind="prefill", B=1, L=L, H=H, D=D, dtype="fp8",
               q=_e4m3(qv), k=_e4m3(kv),
               q_scale=rng.uniform(0.5, 2.0, size=(1, L, H)).astype(np.float32),
               k_scale=rng.uniform(0.5, 2.0, size=(1, L)).astype(np.float32),
               w=rng.standard_normal((1, L, H)).astype(np.float32))
    if not signed:
        inp["w"] = np.abs(inp["w"])
    parity(inp, K, want_scores=True, name=f"fp8 small codes signed={signed}")


@pytest.mark.parametrize("signed", [False, True])
def test_fused_bf16_values_far_from_unit_range(signed):
    """bf16 queries and keys whose magnitudes spread over 2^-20 .. 2^10 per
    query head and per key, with some all-zero keys: the per-token and
    per-key scales the staged bf16 kernel derives (and the exact rescaling of
    both operands) are exercised, and scores and selections match the oracle
    -- with non-negative head weights under the plain tolerance, with signed
    ones under the magnitude-sum tolerance."""
    rng = np.random.default_rng(582)
    L, H, D, K = 700, 64, 128, 64
    qv = rng.standard_normal((1, L, H, D)).astype(np.float32) * np.exp2(rng.integers(-20, 11, size=(1, L, H, 1)))
    kv = rng.standard_normal((1, L, D)).astype(np.float32) * np.exp2(rng.integers(-20, 11, size=(1, L, 1)))
    kv[:, ::53] = 0.0
    w = rng.standard_normal((1, L, H)).astype(np.float32)
    if not signed:
        w = np.abs(w)
    inp = dict(kind="prefill", B=1, L=L, H=H, D=D, dtype="bf16", q=synth.to_bf16_bits(qv), k=synth.to_bf16_bits(kv),
               q_scale=None, k_scale=None, w=w)
    parity(inp, K, want_scores=True, name=f"bf16 wide range signed={signed}")


def test_fused_fp8_mixed_sign_blocks():
    """Signed head weights in every third 8-token block, softmax weights in
    the others: scores and selections match the oracle, the signed rows
    under the magnitude-sum tolerance."""
    inp = synth.prefill_inputs(1, 900, 64, 128, "fp8", seed=581)
    rng = np.random.default_rng(581)
    w = inp["w"].copy()
    for blk in range(0, 900 // 8, 3):  # every third block gets signed weights
        t0 = 8 * blk
        w[0, t0:t0 + 8] = rng.standard_normal((min(8, 900 - t0), 64)).astype(np.float32)
    inp["w"] = w
    parity(inp, 128, want_scores=True, name="fp8 mixed-sign blocks")

"""Pins of the fp64 oracle against things other than itself (CPU only):
the hand-worked 8-token example, the pure-Python brute force, special cases
that reduce to library routines, invariants, cross-call consistency and the
pages' own shape statements.  A final group plants plausible mistakes in the
oracle and checks that these pins catch each of them."""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import brute, indexer

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand8.json")


def hand_inputs(dtype="f32", negate=False, Dpad=None):
    g = json.load(open(GOLD))
    D = g["D"] if Dpad is None else Dpad
    q = np.zeros((1, 8, g["H"], D), np.float32)
    k = np.zeros((1, 8, D), np.float32)
    qh = np.array(g["q_heads"], np.float32) * (-1 if negate else 1)
    q[0, :, :, : g["D"]] = qh[None]
    k[0, :, : g["D"]] = np.array(g["k"], np.float32)
    w = np.broadcast_to(np.array(g["w"], np.float32), (1, 8, g["H"])).copy()
    inp = dict(q=q, k=k, w=w, dtype="f32", q_scale=None, k_scale=None)
    if dtype == "bf16":
        inp.update(q=synth.to_bf16_bits(q), k=synth.to_bf16_bits(k), dtype="bf16")
    elif dtype == "fp8":
        inp.update(q=torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy(),
                   k=torch.from_numpy(k).to(torch.float8_e4m3fn).view(torch.uint8).numpy(),
                   q_scale=np.ones(q.shape[:3], np.float32), k_scale=np.ones(k.shape[:2], np.float32),
                   dtype="fp8")
    return g, inp


def check_hand(mod=indexer):
    """True iff the oracle reproduces every hand-derived number."""
    g, inp = hand_inputs()
    idx, val, I = mod.prefill(inp, 3, want_scores=True)
    ok = np.array_equal(I[0, 7], np.array(g["scores"]))
    for t in range(8):
        ok &= sorted(x for x in idx[0, t] if x >= 0) == g["topk3_sets"][t]
        ok &= all(x == -1 for x in idx[0, t][len(g["topk3_sets"][t]):])
    # masked entries are -inf
    ok &= bool(np.all(np.isneginf(I[0][np.triu_indices(8, 1)])))
    _, inpn = hand_inputs(negate=True)
    idx3, _, In = mod.prefill(inpn, 3, want_scores=True)
    idx4, _, _ = mod.prefill(inpn, 4)
    ok &= np.array_equal(In[0, 7], np.array(g["negated"]["scores"]))
    ok &= sorted(idx3[0, 7].tolist()) == g["negated"]["row7_top3_set"]
    ok &= sorted(idx4[0, 7].tolist()) == g["negated"]["row7_top4_set"]
    return bool(ok)


def test_hand_worked_example():
    assert check_hand()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_hand_example_in_every_format(dtype):
    g, inp = hand_inputs(dtype)
    idx, val, I = indexer.prefill(inp, 3, want_scores=True)
    assert np.array_equal(I[0, 7], np.array(g["scores"]))
    assert sorted(idx[0, 7].tolist()) == [0, 2, 4]


def test_hand_example_zero_padded_to_d64():
    """Padding D from 4 to 64 changes 1/sqrt(D) from 1/2 to 1/8: scores x 1/4."""
    g, inp = hand_inputs(Dpad=64)
    _, _, I = indexer.prefill(inp, 3, want_scores=True)
    assert np.array_equal(I[0, 7], np.array(g["scores"]) / 4)


def random_small(dtype, L, H, D, seed):
    return synth.prefill_inputs(1, L, H, D, dtype, seed)


def check_brute(mod=indexer, cases=(("f32", 9, 3, 5, 11), ("bf16", 12, 2, 4, 12), ("fp8", 10, 3, 6, 13)),
                K=4):
    ok = True
    for dtype, L, H, D, seed in cases:
        inp = random_small(dtype, L, H, D, seed)
        idx, val, I = mod.prefill(inp, K, want_scores=True)
        qs = None if inp["q_scale"] is None else inp["q_scale"][0].tolist()
        ks = None if inp["k_scale"] is None else inp["k_scale"][0].tolist()
        bI, bidx, bval = brute.prefill_one(inp["q"][0].tolist(), inp["k"][0].tolist(),
                                           inp["w"][0].tolist(), dtype, K, qs, ks)
        bI = np.array(bI)
        fin = np.isfinite(bI)
        ok &= np.array_equal(fin, np.isfinite(I[0]))
        ok &= bool(np.allclose(I[0][fin], bI[fin], rtol=1e-12, atol=1e-14))
        ok &= np.array_equal(idx[0], np.array(bidx))
    return bool(ok)


def test_brute_force_agrees():
    assert check_brute()


def test_brute_force_agrees_bf16_queries_fp8_keys():
    """Chunks of bf16 queries against the fp8 cache: the queries and the keys
    are decoded each in its own format (scalar decoders in the brute force)."""
    L, H, D, K = 11, 3, 6, 4
    kin = random_small("fp8", L, H, D, 31)
    qin = random_small("bf16", L, H, D, 32)
    inp = dict(kin, q=qin["q"], q_scale=None, q_dtype="bf16")
    idx, _, I = indexer.prefill(inp, K, want_scores=True)
    bI, bidx, _ = brute.prefill_one(inp["q"][0].tolist(), inp["k"][0].tolist(), inp["w"][0].tolist(), "fp8", K,
                                    None, inp["k_scale"][0].tolist(), q_dtype="bf16")
    bI = np.array(bI)
    fin = np.isfinite(bI)
    assert np.array_equal(fin, np.isfinite(I[0]))
    assert np.allclose(I[0][fin], bI[fin], rtol=1e-12, atol=1e-14)
    assert np.array_equal(idx[0], np.array(bidx))
    # decoding the bf16 queries as fp8 codes would change every score
    wrong = dict(inp, q=(qin["q"] & 0xFF).astype(np.uint8), q_scale=np.ones((1, L, H), np.float32))
    wrong.pop("q_dtype")
    _, _, Iw = indexer.prefill(wrong, K, want_scores=True)
    assert not np.allclose(Iw[0][fin], I[0][fin])


def test_brute_force_tie_heavy():
    inp = synth.tie_heavy_prefill(1, 16, 2, 4, "f32", 7, n_proto=2)
    idx, _, I = indexer.prefill(inp, 5, want_scores=True)
    _, bidx, _ = brute.prefill_one(inp["q"][0].tolist(), inp["k"][0].tolist(), inp["w"][0].tolist(),
                                   "f32", 5)
    assert np.array_equal(idx[0], np.array(bidx))


def test_single_head_unit_weight_is_relu_gemm():
    """H=1, w=1: I = max(q k^T / sqrt(D), 0) -- torch's matmul and relu in fp64."""
    L, D = 40, 16
    inp = random_small("f32", L, 1, D, 21)
    inp["w"][:] = 1.0
    _, _, I = indexer.prefill(inp, 8, want_scores=True)
    qt = torch.from_numpy(inp["q"][0, :, 0].astype(np.float64))
    kt = torch.from_numpy(inp["k"][0].astype(np.float64))
    ref = torch.relu(qt @ kt.T / math.sqrt(D)).numpy()
    tri = np.tril(np.ones((L, L), bool))
    assert np.allclose(I[0][tri], ref[tri], rtol=1e-13, atol=1e-15)


def test_one_hot_weight_picks_one_head():
    L, H, D = 24, 4, 8
    inp = random_small("f32", L, H, D, 22)
    inp["w"][:] = 0.0
    inp["w"][..., 2] = 1.0
    _, _, I = indexer.prefill(inp, 8, want_scores=True)
    qt = torch.from_numpy(inp["q"][0, :, 2].astype(np.float64))
    kt = torch.from_numpy(inp["k"][0].astype(np.float64))
    ref = torch.relu(qt @ kt.T / math.sqrt(D)).numpy()
    tri = np.tril(np.ones((L, L), bool))
    assert np.allclose(I[0][tri], ref[tri], rtol=1e-13)


def test_d1_unit_query_topk_is_stable_argsort():
    """D=1, H=1, q=1, w=1: I[t,s] = max(k_s, 0); the top-k of row t is a
    stable descending argsort of that prefix (numpy's stable sort)."""
    L, K = 50, 7
    rng = np.random.default_rng(5)
    k = np.round(rng.standard_normal((1, L, 1)) * 2).astype(np.float32)  # many exact ties
    inp = dict(q=np.ones((1, L, 1, 1), np.float32), k=k, w=np.ones((1, L, 1), np.float32),
               dtype="f32", q_scale=None, k_scale=None)
    idx, val, _ = indexer.prefill(inp, K)
    for t in range(L):
        v = np.maximum(k[0, : t + 1, 0].astype(np.float64), 0)
        order = np.argsort(-v, kind="stable")[:K]
        exp = np.full(K, -1)
        exp[: order.size] = order
        assert np.array_equal(idx[0, t], exp)


def test_tie_free_topk_matches_torch_topk():
    inp = random_small("f32", 300, 16, 16, 23)
    K = 32
    idx, val, I = indexer.prefill(inp, K, want_scores=True)
    T = torch.from_numpy(I[0])
    tv, ti = torch.topk(T, K, dim=1)
    checked = 0
    for t in range(K, 300):
        srt = np.sort(I[0, t, : t + 1])[::-1]
        if srt[K - 1] == srt[K]:
            continue  # the k-th place is a tie: torch's pick among equals is unspecified
        checked += 1
        assert set(idx[0, t].tolist()) == set(ti[t].tolist())
        assert np.allclose(np.sort(val[0, t]), np.sort(tv[t].numpy()))
    assert checked > 200


def test_invariants_random():
    for dtype, seed in (("f32", 31), ("bf16", 32), ("fp8", 33)):
        L, H, D, K = 96, 8, 32, 20
        inp = random_small(dtype, L, H, D, seed)
        idx, val, I = indexer.prefill(inp, K, want_scores=True)
        I0 = I[0]
        tri = np.tril(np.ones((L, L), bool))
        assert np.all(I0[tri] >= 0)                       # w >= 0  =>  I >= 0
        assert np.all(np.isneginf(I0[~tri]))              # masked s > t
        for t in range(L):
            sel = idx[0, t]
            m = min(K, t + 1)
            assert np.all(sel[:m] >= 0) and np.all(sel[m:] == -1)
            assert np.all(sel[:m] <= t)
            assert len(set(sel[:m].tolist())) == m
            unsel = np.setdiff1d(np.arange(t + 1), sel[:m])
            if unsel.size:
                assert I0[t, sel[:m]].min() >= I0[t, unsel].max()
            assert np.array_equal(val[0, t, :m], I0[t, sel[:m]])


def test_cauchy_schwarz_bound():
    inp = random_small("f32", 64, 4, 16, 34)
    _, _, I = indexer.prefill(inp, 4, want_scores=True)
    q = inp["q"][0].astype(np.float64)
    k = inp["k"][0].astype(np.float64)
    w = inp["w"][0].astype(np.float64)
    nq = np.linalg.norm(q, axis=2)                            # [L,H]
    nk = np.linalg.norm(k, axis=1)                            # [L]
    bound = (w * nq).sum(1)[:, None] * nk[None, :] / 4.0      # sqrt(16) = 4
    tri = np.tril(np.ones((64, 64), bool))
    assert np.all(I[0][tri] <= bound[tri] * (1 + 1e-12))


def test_head_permutation_invariance_and_positive_rescaling():
    inp = random_small("f32", 48, 6, 8, 35)
    K = 10
    idx, val, I = indexer.prefill(inp, K, want_scores=True)
    perm = np.array([3, 1, 5, 0, 2, 4])
    p = dict(inp, q=inp["q"][:, :, perm].copy(), w=inp["w"][:, :, perm].copy())
    idx2, _, I2 = indexer.prefill(p, K, want_scores=True)
    fin = np.isfinite(I)
    assert np.allclose(I[fin], I2[fin], rtol=1e-13) and np.array_equal(idx, idx2)
    r = dict(inp, w=(inp["w"] * 4.0).astype(np.float32), k=(inp["k"] * 2.0).astype(np.float32))
    idx3, _, I3 = indexer.prefill(r, K, want_scores=True)
    assert np.array_equal(idx, idx3)
    assert np.allclose(I3[fin], 8.0 * I[fin], rtol=1e-13)


def test_decode_walkthrough_short_history_returns_all():
    """The decode walkthrough: 8 history tokens and k = 2048 give at most
    min(2048, 8) = 8 positions."""
    d = synth.decode_inputs(1, [8], 4, 32, seed=41, page_size=64, permute=False)
    idx, val = indexer.decode_paged(d, 2048)
    assert sorted(idx[0, :8].tolist()) == list(range(8))
    assert np.all(idx[0, 8:] == -1) and np.all(np.isneginf(val[0, 8:]))


def test_prefill_row_equals_decode_with_prefix_cache():
    """Row t of a prefill equals a decode with ctx = t+1 whose cache holds
    k[0..t] (fp8 keys, bf16 query)."""
    L, H, D, K = 70, 4, 32, 9
    rng = np.random.default_rng(6)
    qb = synth.to_bf16_bits(rng.standard_normal((1, L, H, D)).astype(np.float32))
    kc, ks = synth.quantize_fp8_rows(rng.standard_normal((1, L, D)).astype(np.float32))
    w = synth.softmax_weights(rng.standard_normal((1, L, H)))
    # prefill with fp8 keys needs fp8 queries; compare through scores instead
    for t in (0, 5, 40, 69):
        ctx = t + 1
        npg = -(-ctx // 16)
        kcp = np.zeros((npg, 16, D), np.uint8)
        ksp = np.ones((npg, 16), np.float32)
        kcp.reshape(-1, D)[:ctx] = kc[0, :ctx]
        ksp.reshape(-1)[:ctx] = ks[0, :ctx]
        d = dict(q=qb[0, t:t + 1], w=w[0, t:t + 1], k_cache=kcp, k_scale=ksp,
                 block_table=np.arange(npg, dtype=np.int32)[None], context_lens=np.array([ctx]),
                 page_size=16, q_dtype="bf16")
        I_dec = indexer.decode_scores(d, 0)
        from oracle import formats
        qd = formats.decode(qb[0, t], "bf16")
        kd = formats.decode(kc[0, :ctx], "fp8", ks[0, :ctx])
        ref = (w[0, t].astype(np.float64)[:, None] * np.maximum(qd @ kd.T / math.sqrt(D), 0)).sum(0)
        assert np.allclose(I_dec, ref, rtol=1e-13)
        # brute force on a couple of positions
        for s in (0, t):
            (bi, bv), vals = brute.decode_one(qb[0, t].tolist(), w[0, t].tolist(), kcp.tolist(),
                                              ksp.tolist(), d["block_table"][0].tolist(), ctx, 16,
                                              K, "bf16")
            assert math.isclose(vals[s], I_dec[s], rel_tol=1e-12, abs_tol=1e-15)
            assert bi == indexer.select_topk(I_dec, ctx, K)[0].tolist()


def test_paged_permutation_matches_identity_layout():
    d1 = synth.decode_inputs(3, [100, 64, 130], 4, 32, seed=44, page_size=16, permute=True)
    # rebuild the same logical caches in identity layout
    B, ps = 3, 16
    rows_c, rows_s, bt = [], [], np.zeros_like(d1["block_table"])
    off = 0
    for b in range(B):
        n = -(-int(d1["context_lens"][b]) // ps)
        for j in range(n):
            p = d1["block_table"][b, j]
            rows_c.append(d1["k_cache"][p])
            rows_s.append(d1["k_scale"][p])
            bt[b, j] = off + j
        off += n
    d2 = dict(d1, k_cache=np.stack(rows_c), k_scale=np.stack(rows_s), block_table=bt)
    i1, v1 = indexer.decode_paged(d1, 50)
    i2, v2 = indexer.decode_paged(d2, 50)
    assert np.array_equal(i1, i2) and np.array_equal(v1, v2)


def test_tutorial_listing_shapes():
    """The tutorial's example: batch 2, L = 1024, top_k = 128 gives index
    shape (2, 1024, 128) and score shape (2, 1024, 1024)."""
    inp = synth.prefill_inputs(2, 1024, 2, 8, "f32", 45)
    idx, val, I = indexer.prefill(inp, 128, want_scores=True)
    assert idx.shape == (2, 1024, 128) and I.shape == (2, 1024, 1024)
    assert np.all(idx[:, :127, -1] == -1) and np.all(idx[:, 127:] >= 0)


def test_topk_rows_handles_signed_zero_and_ties():
    row = np.array([[0.0, -0.0, 1.0, -0.0, 0.0, 1.0, -1.0]], np.float32)
    idx, val = indexer.topk_rows(row, None, 4)
    assert idx[0].tolist() == [2, 5, 0, 1]
    idx, val = indexer.topk_rows(row, [3], 5)
    assert idx[0].tolist() == [2, 0, 1, -1, -1]


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant must be caught by at least one pin above.
# ---------------------------------------------------------------------------

def _mutant_scores(kind):
    orig = indexer._scores_block

    def f(qd_rows, kd, w_rows):
        R, H, D = qd_rows.shape
        S = np.matmul(qd_rows.reshape(R * H, D), kd.T).reshape(R, H, kd.shape[0])
        if kind == "no_relu":
            r = S / np.sqrt(D)
        elif kind == "no_scale":
            r = np.maximum(S, 0)
        elif kind == "relu_after_sum":
            return np.maximum(np.einsum("rh,rhn->rn", w_rows, S / np.sqrt(D)), 0)
        elif kind == "unweighted":
            r = np.maximum(S / np.sqrt(D), 0)
            return r.sum(1)
        elif kind == "abs":
            r = np.abs(S / np.sqrt(D))
        else:
            raise ValueError(kind)
        return np.einsum("rh,rhn->rn", w_rows, r)
    return orig, f


@pytest.mark.parametrize("kind", ["no_relu", "no_scale", "relu_after_sum", "unweighted", "abs"])
def test_pins_catch_planted_score_mistakes(monkeypatch, kind):
    orig, f = _mutant_scores(kind)
    monkeypatch.setattr(indexer, "_scores_block", f)
    assert not (check_hand() and check_brute())


def test_pins_catch_reversed_tie_rule(monkeypatch):
    def bad(row, n_valid, K):
        v = np.asarray(row[:n_valid], np.float64)
        s = np.arange(n_valid)
        order = np.lexsort((-s, -v))
        m = min(K, n_valid)
        idx = np.full(K, -1, np.int32)
        val = np.full(K, -np.inf)
        idx[:m] = order[:m]
        val[:m] = v[order[:m]]
        return idx, val
    monkeypatch.setattr(indexer, "select_topk", bad)
    assert not check_hand()


def test_pins_catch_strict_causal_mask(monkeypatch):
    orig = indexer.prefill_scores

    def strict(*a, **kw):
        out = orig(*a, **kw)
        rows = kw.get("rows")
        rows = np.arange(out.shape[0]) if rows is None else np.asarray(rows)
        out[np.arange(rows.size), rows] = -np.inf
        return out
    monkeypatch.setattr(indexer, "prefill_scores", strict)
    assert not check_hand()

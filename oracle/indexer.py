"""Vectorised fp64 oracle of the lightning indexer and its top-k selector
(test infrastructure; see the package docstring).

Definition followed, step by step, in the order the pages give it:

1. Decode every stored input to fp64 (``formats.decode``).
2. For each query token t and index head i, dot the head's query with the
   ONE key shared by all heads of history token s:  S[t,i,s] = q[t,i] . k[s].
   (Lightning Indexer explained, section 4 "scoring formula": multi-head is on
   the query side only, the key is row s of the indexer cache; Study MLA
   Indexer, data flow: one d_idx-wide key per token.)
3. Scale by 1/sqrt(D) and apply ReLU:  r = max(S / sqrt(D), 0).
   (From principle to code -- DeepSeek-V3.2 lightning indexer, section 2.1
   "core formula": the scaled dot product goes through ReLU; Study MLA
   Indexer, data flow: logits carry the 1/sqrt(d_idx) factor.  The second
   page's formula omits the factor; the reading taken is that it is present,
   inside the ReLU.)
4. Weighted sum over heads:  I[t,s] = sum_i w[t,i] * r[t,i,s]
   (same formula; w is an input here).
5. History set.  Prefill: s <= t (the tutorial listing's inclusive lower
   triangular mask; the prose says s < t -- the reading taken is s <= t, the
   current token's key having been written to the cache before scoring as
   the Study MLA Indexer page orders it).  Decode: the query sits at
   position ctx-1 and sees s in [0, ctx).  Masked entries are -inf in a
   materialised score row (the listing's masked_fill with -inf).
6. Top-k: among the valid s, order by (I desc, s asc) with a full sort and
   keep the first min(k, n_valid); pad the rest with -1 (the walkthrough of
   a decode step: at most min(2048, L) positions come back).  Ties go to the
   lower index.  Equal values compare equal in this sort, so -0.0 and +0.0
   tie.

numpy's matmul is the only library step (the dot products of step 2).
"""
from __future__ import annotations

import numpy as np

from .formats import decode

_BLOCK_BYTES = 1 << 28  # bound on the fp64 S block held at once


def _scores_block(qd_rows: np.ndarray, kd: np.ndarray, w_rows: np.ndarray) -> np.ndarray:
    """qd_rows [R,H,D], kd [N,D], w_rows [R,H]  ->  I [R,N] (steps 2-4, unmasked)."""
    R, H, D = qd_rows.shape
    S = np.matmul(qd_rows.reshape(R * H, D), kd.T).reshape(R, H, kd.shape[0])  # step 2
    z = S / np.sqrt(np.float64(D))                                              # step 3
    r = np.maximum(z, 0.0)                                                      # step 3
    return np.einsum("rh,rhn->rn", w_rows, r)                                   # step 4


def prefill_scores(q, k, w, dtype: str, q_scale=None, k_scale=None, rows=None, q_dtype=None) -> np.ndarray:
    """Score rows of ONE sequence.

    q [L,H,D], k [L,D], w [L,H] as stored (see ``formats.decode``); q_scale
    [L,H] and k_scale [L] for fp8.  ``q_dtype`` is the queries' format when
    it differs from the keys' (bf16 queries of a chunk scored against an fp8
    key cache: each side decoded on its own, step 1).  Returns fp64
    [len(rows), L] with -inf at s > t (all rows when ``rows`` is None).
    """
    L, H, D = q.shape
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    kd = decode(k, dtype, k_scale)
    wd = np.asarray(w, dtype=np.float32).astype(np.float64)
    out = np.full((rows.size, L), -np.inf, dtype=np.float64)
    per_row = max(1, H * L * 8)
    blk = max(1, _BLOCK_BYTES // per_row)
    for a in range(0, rows.size, blk):
        rr = rows[a:a + blk]
        n = int(rr.max()) + 1
        qd = decode(q[rr], q_dtype or dtype, None if q_scale is None else q_scale[rr])
        I = _scores_block(qd, kd[:n], wd[rr])
        s = np.arange(n)
        I = np.where(s[None, :] <= rr[:, None], I, -np.inf)                    # step 5
        out[a:a + blk, :n] = I
    return out


def select_topk(row: np.ndarray, n_valid: int, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Step 6 for one row whose first ``n_valid`` entries are the valid
    positions.  Returns (idx int32 [K], val fp64 [K]); padding is -1 / -inf."""
    v = np.asarray(row[:n_valid], dtype=np.float64)
    s = np.arange(n_valid)
    order = np.lexsort((s, -v))          # primary key -I, secondary key s
    m = min(K, n_valid)
    idx = np.full(K, -1, dtype=np.int32)
    val = np.full(K, -np.inf, dtype=np.float64)
    idx[:m] = order[:m]
    val[:m] = v[order[:m]]
    return idx, val


def prefill(inp: dict, K: int, rows=None, want_scores: bool = False):
    """Oracle of one prefill call over every batch element.

    ``inp`` holds q [B,L,H,D], k [B,L,D], w [B,L,H] (+ q_scale [B,L,H],
    k_scale [B,L] for fp8) and "dtype" (+ "q_dtype" when the queries' format
    differs from the keys').  Returns (idx [B,R,K] int32,
    val [B,R,K] fp64, scores [B,R,L] fp64 or None) for the R requested rows.
    """
    q, k, w, dt = inp["q"], inp["k"], inp["w"], inp["dtype"]
    B, L = q.shape[0], q.shape[1]
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    idx = np.empty((B, rows.size, K), dtype=np.int32)
    val = np.empty((B, rows.size, K), dtype=np.float64)
    scores = np.empty((B, rows.size, L), dtype=np.float64) if want_scores else None
    qs, ks = inp.get("q_scale"), inp.get("k_scale")
    for b in range(B):
        I = prefill_scores(q[b], k[b], w[b], dt,
                           None if qs is None else qs[b], None if ks is None else ks[b], rows,
                           q_dtype=inp.get("q_dtype"))
        for j, t in enumerate(rows):
            idx[b, j], val[b, j] = select_topk(I[j], int(t) + 1, K)
        if want_scores:
            scores[b] = I
    return idx, val, scores


def decode_scores(inp: dict, b: int) -> np.ndarray:
    """Scores of decode query b over its context, fp64 [ctx_b].

    Logical position s lives in page block_table[b][s // page_size] at slot
    s % page_size of the pool; its value is the fp8 code times that token's
    scale."""
    ps = inp["page_size"]
    ctx = int(inp["context_lens"][b])
    s = np.arange(ctx)
    pages = inp["block_table"][b, s // ps].astype(np.int64)
    slots = s % ps
    kd = decode(inp["k_cache"][pages, slots], "fp8", inp["k_scale"][pages, slots])
    qd = decode(inp["q"][b], inp.get("q_dtype", "bf16"))
    wd = np.asarray(inp["w"][b], dtype=np.float32).astype(np.float64)
    return _scores_block(qd[None], kd, wd[None])[0]


def decode_paged(inp: dict, K: int, queries=None):
    """Oracle of one paged decode call.  Returns (idx [Q,K] int32, val [Q,K])."""
    B = inp["q"].shape[0]
    queries = range(B) if queries is None else queries
    out_i, out_v = [], []
    for b in queries:
        I = decode_scores(inp, b)
        i, v = select_topk(I, I.size, K)
        out_i.append(i)
        out_v.append(v)
    return np.stack(out_i), np.stack(out_v)


def topk_rows(scores: np.ndarray, row_len, K: int):
    """Top-k of each row of a plain score matrix (the standalone selector):
    row r's valid entries are its first row_len[r] columns."""
    R, C = scores.shape
    row_len = np.full(R, C) if row_len is None else np.asarray(row_len)
    idx = np.empty((R, K), dtype=np.int32)
    val = np.empty((R, K), dtype=np.float64)
    for r in range(R):
        idx[r], val[r] = select_topk(scores[r], int(row_len[r]), K)
    return idx, val

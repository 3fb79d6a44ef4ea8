"""(Test infrastructure.)  Parity rules between the HIP library's outputs and the fp64 oracle.

Scores: |g - o| <= max(1e-4, 1e-3 * |o|) per element, -inf exactly where
the oracle masks.

Top-k sets (one row, n_valid valid positions, m = min(k, n_valid)):
  (i)   the first m slots hold valid positions, the rest are -1 (score -inf);
  (ii)  no position repeats;
  (iii) against the oracle's set O (by score desc, position asc) with
        tau = O's m-th score, every position in the symmetric difference
        of the two sets has an oracle score within max(1e-4, 1e-3|tau|) of
        tau -- i.e. only near-ties at the cut may swap;
  (iv)  each returned score matches the oracle's score of that position
        under the score rule.
When n_valid <= k the set must be all valid positions.

Signed head weights: every rule above takes, where given, the magnitude sum
M = sum_h |w_h * q_scale_h| * ReLU(q_h . k / sqrt(D)) of each score into its
tolerance tol = max(1e-4, 1e-3 |o|, 1e-3 M).  M is the score itself when the
weights are non-negative (then nothing changes); with mixed signs a score
can cancel far below M, and the rounding of the head terms of any
floating-point evaluation is bounded relative to M, not to the cancelled
result.  Tolerances then differ from position to position, so rule (iii)
reads per position: the returned set must be the top m of some score vector
within each position's tolerance of the oracle's, i.e. the lowest o + tol
over the returned positions is at least the highest o - tol over the
others.
"""
from __future__ import annotations

import numpy as np

ABS_TOL = 1e-4
REL_TOL = 1e-3


def score_tol(o, mag=None):
    t = np.maximum(ABS_TOL, REL_TOL * np.abs(o))
    if mag is not None:
        t = np.maximum(t, REL_TOL * np.abs(np.asarray(mag, np.float64)))
    return t


def check_scores(g: np.ndarray, o: np.ndarray, what: str = "scores", mag=None) -> None:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    mask_o = np.isneginf(o)
    bad_mask = mask_o != np.isneginf(g)
    if bad_mask.any():
        i = np.argwhere(bad_mask)[0]
        raise AssertionError(f"{what}: -inf mismatch at {tuple(i)}: gpu={g[tuple(i)]} oracle={o[tuple(i)]}")
    fin = ~mask_o
    err = np.abs(g[fin] - o[fin])
    tol = score_tol(o[fin], None if mag is None else np.asarray(mag, np.float64)[fin])
    if np.any(~(err <= tol)):
        j = np.argmax(err / tol)
        raise AssertionError(f"{what}: {np.sum(~(err <= tol))} of {err.size} outside tolerance; worst gpu="
                             f"{g[fin][j]!r} oracle={o[fin][j]!r} err={err[j]:.3g} tol={tol[j]:.3g}")


def check_topk_row(g_idx, g_val, o_row, n_valid: int, K: int, where: str = "", mag_row=None) -> dict:
    """o_row: oracle fp64 scores of positions [0, n_valid); mag_row: their
    magnitude sums (signed weights) or None.  Returns stats."""
    g_idx = np.asarray(g_idx, np.int64)
    m = min(K, n_valid)
    head, tail = g_idx[:m], g_idx[m:]
    if np.any(tail != -1):
        raise AssertionError(f"{where}: expected -1 padding after {m} entries, got {tail[tail != -1][:5]}")
    if np.any((head < 0) | (head >= n_valid)):
        raise AssertionError(f"{where}: invalid positions {head[(head < 0) | (head >= n_valid)][:5]}")
    if np.unique(head).size != m:
        raise AssertionError(f"{where}: duplicate positions")
    if g_val is not None:
        g_val = np.asarray(g_val, np.float64)
        if np.any(~np.isneginf(g_val[m:])):
            raise AssertionError(f"{where}: padding scores must be -inf")
        check_scores(g_val[:m], o_row[head], what=f"{where} selected scores",
                     mag=None if mag_row is None else mag_row[head])
    if n_valid <= K:
        return dict(swaps=0)
    s = np.arange(n_valid)
    order = np.lexsort((s, -o_row[:n_valid]))
    O = order[:m]
    tau = o_row[O[-1]]
    diff = np.setxor1d(head, O)
    if mag_row is None:
        tol = max(ABS_TOL, REL_TOL * abs(tau))
        far = diff[np.abs(o_row[diff] - tau) > tol]
    else:
        # per-position tolerances: some scores within them must rank the
        # returned set first
        ov = o_row[:n_valid]
        tv = score_tol(ov, np.asarray(mag_row, np.float64)[:n_valid])
        sel = np.zeros(n_valid, bool)
        sel[head] = True
        lo_in = np.min(ov[sel] + tv[sel])
        hi_out = np.max(ov[~sel] - tv[~sel])
        far = diff[(sel[diff] & (ov[diff] + tv[diff] < hi_out)) | (~sel[diff] & (ov[diff] - tv[diff] > lo_in))]
    if far.size:
        raise AssertionError(f"{where}: {far.size} positions differ from the oracle's set beyond the tie "
                             f"tolerance; e.g. s={far[0]} score={o_row[far[0]]!r} tau={tau!r}")
    return dict(swaps=int(diff.size // 2))


def check_topk_rows(g_idx, g_val, o_scores, n_valid, K, where="", mag=None) -> int:
    swaps = 0
    for r in range(g_idx.shape[0]):
        st = check_topk_row(g_idx[r], None if g_val is None else g_val[r], o_scores[r], int(n_valid[r]), K,
                            where=f"{where} row {r}", mag_row=None if mag is None else mag[r])
        swaps += st["swaps"]
    return swaps

"""Scalar pure-Python twin of ``indexer`` for tiny inputs (test infrastructure).

It restates the same definition -- I[t,s] = sum_i w[t,i] * max(q[t,i].k[s]/sqrt(D), 0)
over s <= t, then the k largest by (score desc, index asc), -1 padded -- with
explicit loops and its own scalar decoders (``struct`` for bf16, ``math.ldexp``
for fp8), so a slip in the vectorised code (a transposed operand, a dropped
term, a wrong mask or tie rule) shows up as a disagreement.  Only for L <= 64
or so: it is O(L^2 * H * D) Python.
"""
from __future__ import annotations

import math
import struct


def fp8_value(code: int) -> float:
    code &= 0xFF
    neg = code >> 7
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        v = math.ldexp(m, -9)               # m/8 * 2^(1-7)
    else:
        v = math.ldexp(8 + m, e - 10)       # (1 + m/8) * 2^(e-7)
    return -v if neg else v


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _val(x, dtype: str, scale=None) -> float:
    if dtype == "f32":
        return float(x)
    if dtype == "bf16":
        return bf16_value(int(x))
    return fp8_value(int(x)) * float(scale)


def score(q_t, k_s, w_t, dtype, qs_t=None, ks_s=None, q_dtype=None) -> float:
    """One I[t,s]: q_t [H][D], k_s [D], w_t [H] as stored (queries in
    q_dtype when it is given, else in the keys' dtype)."""
    H, D = len(q_t), len(k_s)
    kv = [_val(k_s[c], dtype, ks_s) for c in range(D)]
    total = 0.0
    for i in range(H):
        dot = 0.0
        for c in range(D):
            dot += _val(q_t[i][c], q_dtype or dtype, None if qs_t is None else qs_t[i]) * kv[c]
        total += float(w_t[i]) * max(dot / math.sqrt(D), 0.0)
    return total


def topk(values: list, K: int) -> tuple[list, list]:
    """values[s] for the valid s, in index order -> (idx, val) with -1 padding."""
    order = sorted(range(len(values)), key=lambda s: (-values[s], s))[:K]
    idx = order + [-1] * (K - len(order))
    val = [values[s] for s in order] + [-math.inf] * (K - len(order))
    return idx, val


def prefill_one(q, k, w, dtype, K, q_scale=None, k_scale=None, q_dtype=None):
    """One sequence: q [L][H][D], k [L][D], w [L][H].  Returns
    (I as list of rows with -inf at s > t, idx rows, val rows)."""
    L = len(q)
    I, idx, val = [], [], []
    for t in range(L):
        row = []
        for s in range(L):
            if s <= t:
                row.append(score(q[t], k[s], w[t], dtype,
                                 None if q_scale is None else q_scale[t],
                                 None if k_scale is None else k_scale[s], q_dtype))
            else:
                row.append(-math.inf)
        I.append(row)
        i, v = topk(row[: t + 1], K)
        idx.append(i)
        val.append(v)
    return I, idx, val


def decode_one(q_b, w_b, k_cache, k_scale, bt_b, ctx, page_size, K, q_dtype="bf16"):
    """One decode query over its paged context."""
    H = len(q_b)
    D = len(q_b[0])
    vals = []
    for s in range(ctx):
        p, slot = int(bt_b[s // page_size]), s % page_size
        kv = [fp8_value(int(k_cache[p][slot][c])) * float(k_scale[p][slot]) for c in range(D)]
        total = 0.0
        for i in range(H):
            dot = 0.0
            for c in range(D):
                dot += _val(q_b[i][c], q_dtype) * kv[c]
            total += float(w_b[i]) * max(dot / math.sqrt(D), 0.0)
        vals.append(total)
    return topk(vals, K), vals

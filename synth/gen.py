"""Seeded input generators for the five indexer workloads.

Byte formats produced (these are what both the oracle and the HIP library read):

* fp32   : IEEE binary32, numpy float32.
* bf16   : the upper 16 bits of binary32 after round-to-nearest-even, stored
           as uint16 (torch's CPU cast does the rounding).
* fp8    : OCP FP8 E4M3FN codes stored as uint8, produced from an fp32 source
           row x by  scale = absmax(x) / 448  (1.0 when the row is all zero),
           code = e4m3(clamp(x / scale, -448, 448))  with round-to-nearest-even
           (torch's CPU cast does the rounding; the clamp makes it saturating so
           no NaN code is ever emitted).  The value a code stands for is
           decoded_code * scale.

Random numbers come from numpy's PCG64 generator seeded with the workload
number unless a seed is given.  Draw order is fixed per generator and written
next to each function.

Nothing here evaluates the indexer: no dot product, ReLU, head reduction,
masking or selection.
"""
from __future__ import annotations

import numpy as np
import torch

FP8_MAX = 448.0

# The five workloads: tiny fp32 prefill, bf16 prefill with planted needles,
# fp8 prefill at 32K, contiguous fp8 decode and paged fp8 decode.
CONFIGS = {
    1: dict(kind="prefill", B=1, L=256, H=4, D=32, topk=16, dtype="f32"),
    2: dict(kind="prefill", B=1, L=8192, H=64, D=128, topk=2048, dtype="bf16", needles=True),
    3: dict(kind="prefill", B=1, L=32768, H=64, D=128, topk=2048, dtype="fp8"),
    4: dict(kind="decode", B=64, ctx="fixed", ctx_len=131072, H=64, D=128, topk=2048,
            page_size=64, permute=False),
    5: dict(kind="decode", B=128, ctx="uniform", ctx_lo=4096, ctx_hi=131072, H=64, D=128,
            topk=2048, page_size=64, permute=True),
}

_CHUNK_ROWS = 1 << 20  # rows quantised per chunk, to bound host memory


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float32 values (a widening cast, used only to
    form the needle direction from already-rounded queries)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def quantize_fp8_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row (last axis) absmax/448 scaling and saturating RNE to OCP E4M3FN.

    Returns (codes uint8 with x's shape, scales float32 with x.shape[:-1]).
    Rows are processed in chunks so a 1e9-element source needs bounded memory.
    """
    x = np.asarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    n = flat.shape[0]
    codes = np.empty((n, D), dtype=np.uint8)
    scales = np.empty((n,), dtype=np.float32)
    for r0 in range(0, n, _CHUNK_ROWS):
        r1 = min(n, r0 + _CHUNK_ROWS)
        t = torch.from_numpy(flat[r0:r1])
        amax = t.abs().amax(dim=1)
        sc = amax / FP8_MAX
        sc = torch.where(amax > 0, sc, torch.ones_like(sc))
        y = torch.clamp(t / sc[:, None], -FP8_MAX, FP8_MAX)
        codes[r0:r1] = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        scales[r0:r1] = sc.numpy()
    return codes.reshape(*lead, D), scales.reshape(lead)


def softmax_weights(logits: np.ndarray) -> np.ndarray:
    """Head weights as a softmax over the last axis (fp64, stored as fp32).

    The pages make the head weights a softmax-normalised projection of the
    query token; here the logits are random draws standing in for that
    projection."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def prefill_inputs(B: int, L: int, H: int, D: int, dtype: str, seed: int,
                   needles: bool = False, needle_block: int = 64, n_needles: int = 32,
                   topk: int | None = None) -> dict:
    """Inputs of one prefill call.

    Draw order: q source, k source, w logits, then (bf16 with needles only)
    per query block in increasing order: needle positions, then needle noise.

    Needles: for each block of `needle_block` query tokens, q-mean is the mean
    of the block's bf16 queries over its tokens and heads; `n_needles`
    distinct positions are drawn uniformly from the not-yet-planted positions
    in [0, block_end) and their keys are replaced by bf16(0.5*q-mean + N(0,1)).
    """
    rng = make_rng(seed)
    out = dict(kind="prefill", B=B, L=L, H=H, D=D, dtype=dtype, seed=seed, topk=topk)
    qsrc = _normal(rng, (B, L, H, D))
    ksrc = _normal(rng, (B, L, D))
    out["w"] = softmax_weights(_normal(rng, (B, L, H)).astype(np.float64))
    if dtype == "f32":
        out["q"], out["k"] = qsrc, ksrc
        out["q_scale"] = out["k_scale"] = None
    elif dtype == "bf16":
        out["q"] = to_bf16_bits(qsrc)
        del qsrc
        kb = to_bf16_bits(ksrc)
        if needles:
            qf = bf16_bits_to_f32(out["q"])
            planted_pos = []
            for b in range(B):
                planted = np.zeros(L, dtype=bool)
                for blk0 in range(0, L, needle_block):
                    blk1 = min(L, blk0 + needle_block)
                    qmean = qf[b, blk0:blk1].astype(np.float64).mean(axis=(0, 1))
                    avail = np.flatnonzero(~planted[:blk1])
                    m = min(n_needles, avail.size)
                    pos = np.sort(rng.choice(avail, size=m, replace=False))
                    noise = rng.standard_normal(size=(m, D))
                    planted[pos] = True
                    kb[b, pos] = to_bf16_bits((0.5 * qmean[None, :] + noise).astype(np.float32))
                    planted_pos.append((b, blk0, pos))
            out["needles"] = planted_pos
        out["k"] = kb
        out["q_scale"] = out["k_scale"] = None
    elif dtype == "fp8":
        out["q"], out["q_scale"] = quantize_fp8_rows(qsrc)
        del qsrc
        out["k"], out["k_scale"] = quantize_fp8_rows(ksrc)
    else:
        raise ValueError(dtype)
    return out


def tie_heavy_prefill(B: int, L: int, H: int, D: int, dtype: str, seed: int,
                      n_proto: int = 4) -> dict:
    """Prefill inputs whose keys repeat a few prototype vectors, so many
    (t, s) scores tie exactly.  Draw order: q source, prototype keys,
    prototype choice per position, w logits."""
    rng = make_rng(seed)
    qsrc = _normal(rng, (B, L, H, D))
    protos = _normal(rng, (n_proto, D))
    choice = rng.integers(0, n_proto, size=(B, L))
    ksrc = protos[choice]
    w = softmax_weights(_normal(rng, (B, L, H)).astype(np.float64))
    out = dict(kind="prefill", B=B, L=L, H=H, D=D, dtype=dtype, seed=seed, w=w)
    if dtype == "f32":
        out.update(q=qsrc, k=ksrc, q_scale=None, k_scale=None)
    elif dtype == "bf16":
        out.update(q=to_bf16_bits(qsrc), k=to_bf16_bits(ksrc), q_scale=None, k_scale=None)
    else:
        q, qs = quantize_fp8_rows(qsrc)
        k, ks = quantize_fp8_rows(ksrc)
        out.update(q=q, q_scale=qs, k=k, k_scale=ks)
    return out


def decode_inputs(B: int, ctx_lens, H: int, D: int, seed: int, page_size: int = 64,
                  permute: bool = True, q_dtype: str = "bf16", extra_pages: int = 0,
                  max_pages_per_seq: int | None = None, topk: int | None = None) -> dict:
    """Inputs of one paged decode call.

    `ctx_lens` is either a list of B context lengths or a (lo, hi) pair, in
    which case lengths are drawn uniformly from the integers lo..hi inclusive.

    Draw order: context lengths (if drawn), q source, w logits, page
    permutation (if permute), then the key pool in page order.

    The pool holds sum_b ceil(ctx_b / page_size) pages (+ extra_pages spare
    pages that no query references).  Without permutation query b owns a
    contiguous run of pages; with it, a seeded permutation of the page ids is
    dealt to the queries in order.  Block-table entries past a query's last
    page are 0 and never read.  Every token of the pool, used or not, gets an
    N(0,1) key quantised to fp8 with its own absmax/448 scale.
    """
    rng = make_rng(seed)
    if isinstance(ctx_lens, tuple):
        lo, hi = ctx_lens
        ctx = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        ctx = np.asarray(ctx_lens, dtype=np.int32)
        assert ctx.shape == (B,)
    qsrc = _normal(rng, (B, H, D))
    w = softmax_weights(_normal(rng, (B, H)).astype(np.float64))
    npages = (ctx.astype(np.int64) + page_size - 1) // page_size
    pool = int(npages.sum()) + extra_pages
    ids = rng.permutation(pool).astype(np.int32) if permute else np.arange(pool, dtype=np.int32)
    mpp = int(npages.max()) if max_pages_per_seq is None else max_pages_per_seq
    bt = np.zeros((B, mpp), dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(npages[b])
        bt[b, :n] = ids[off:off + n]
        off += n
    kc = np.empty((pool, page_size, D), dtype=np.uint8)
    ks = np.empty((pool, page_size), dtype=np.float32)
    pages_per_chunk = max(1, _CHUNK_ROWS // page_size)
    for p0 in range(0, pool, pages_per_chunk):
        p1 = min(pool, p0 + pages_per_chunk)
        c, s = quantize_fp8_rows(_normal(rng, (p1 - p0, page_size, D)))
        kc[p0:p1] = c
        ks[p0:p1] = s
    out = dict(kind="decode", B=B, H=H, D=D, seed=seed, page_size=page_size,
               context_lens=ctx, block_table=bt, k_cache=kc, k_scale=ks, w=w,
               max_pages_per_seq=mpp, num_pages=pool, topk=topk)
    if q_dtype == "bf16":
        out["q"] = to_bf16_bits(qsrc)
    else:
        out["q"] = qsrc
    out["q_dtype"] = q_dtype
    return out


def config_inputs(n: int, seed: int | None = None) -> dict:
    """Full-size inputs of workload n (1..5), seeded with n unless given."""
    c = CONFIGS[n]
    s = n if seed is None else seed
    if c["kind"] == "prefill":
        d = prefill_inputs(c["B"], c["L"], c["H"], c["D"], c["dtype"], s,
                           needles=c.get("needles", False), topk=c["topk"])
    else:
        ctx = [c["ctx_len"]] * c["B"] if c["ctx"] == "fixed" else (c["ctx_lo"], c["ctx_hi"])
        d = decode_inputs(c["B"], ctx, c["H"], c["D"], s, page_size=c["page_size"],
                          permute=c["permute"], topk=c["topk"],
                          max_pages_per_seq=(c.get("ctx_len") or c.get("ctx_hi")) // c["page_size"])
    d["config"] = n
    return d


def causal_pairs(L: int) -> int:
    """Number of (t, s) pairs with 0 <= s <= t < L."""
    return L * (L + 1) // 2


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


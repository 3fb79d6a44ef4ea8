"""The indexer K-cache write path, oracle side: per-token FP8 quantisation of
new keys and their append into the paged cache.  Test infrastructure: only
tests/, the smoke check and the benchmark's CPU baseline use it.

What the pages fix: the indexer keeps its own key cache, in FP8; each
token's key is appended to it once, when that token is processed, and later
steps only read it; the cache is updated before the scoring decision
(Lightning Indexer explained, sections 2.1 and 2.4 of the decode walkthrough
and section 5 "Indexer-Cache"; Study MLA Indexer, the data-flow diagram,
whose key path ends in an FP8 quantisation, and the notes on its two
caches).  What they leave open, and the readings taken here:

* FP8 flavour: OCP E4M3FN, as for every stored key (formats.py).
* Scaling: one fp32 scale per token, absmax(key) / 448 computed in fp32
  (1.0 for an all-zero key), so the key's largest magnitude lands on the
  largest finite code.  The stored value of element d is
  decode(code_d) * scale.
* Rounding: code_d is the E4M3FN value nearest to the fp32 quotient
  x_d / scale (an IEEE binary32 division), ties to the even code (the one
  whose mantissa ends in 0), magnitudes above 448 saturated to 448, the sign
  kept (so -0.0 gives 0x80).
* Placement: the token of sequence b at position p goes to page
  block_table[b][p // page_size], slot p % page_size: the layout the paged
  decode reads.  A token whose sequence id lies outside [0, B) (B rows of
  the block table; -1 marks padding) or whose position lies outside
  [0, max_pages_per_seq * page_size) is not written.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, fp8_e4m3_to_f64

E4M3_MAX = 448.0

# The 127 non-negative finite codes 0x00 .. 0x7E, in increasing value.
_CODES = np.arange(0, 0x7F, dtype=np.int64)
_VALUES = fp8_e4m3_to_f64(_CODES.astype(np.uint8))


def encode_e4m3(y) -> np.ndarray:
    """Values -> E4M3FN codes: the nearest finite value, ties to the even
    code, magnitudes beyond 448 saturated, the sign bit copied from y."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.clip(np.searchsorted(_VALUES, mag, side="left"), 0, len(_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_VALUES) - 1)
    d_lo = mag - _VALUES[lo]
    d_hi = _VALUES[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_CODES[hi] % 2 == 0))
    code = np.where(take_hi, _CODES[hi], _CODES[lo])
    return (code | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def key_rows_to_f32(keys: np.ndarray, dtype: str) -> np.ndarray:
    """New keys as stored by the caller ("f32": float32, "bf16": uint16 bit
    patterns) -> float32 (exact for both)."""
    if dtype == "f32":
        return np.asarray(keys, dtype=np.float32)
    if dtype == "bf16":
        return bf16_to_f64(keys).astype(np.float32)
    raise ValueError(f"unknown key dtype {dtype!r}")


def quantize_keys(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """float32 keys [..., D] -> (E4M3FN codes [..., D], fp32 scales [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quotient = (x / scale[..., None]).astype(np.float32)  # binary32 division, as stated above
    return encode_e4m3(quotient), scale


def kcache_append(k_cache: np.ndarray, k_scale: np.ndarray, keys: np.ndarray, dtype: str,
                  seq_ids: np.ndarray, positions: np.ndarray, block_table: np.ndarray,
                  page_size: int = 64) -> tuple[np.ndarray, np.ndarray]:
    """Returns copies of (k_cache [pages][page_size][D] uint8,
    k_scale [pages][page_size] fp32) with the new keys written.  Keys are
    taken in order, so of two tokens with the same (sequence, position) the
    later one stays (the GPU leaves that case unspecified)."""
    cache = np.array(k_cache, dtype=np.uint8, copy=True)
    scales = np.array(k_scale, dtype=np.float32, copy=True)
    codes, sc = quantize_keys(key_rows_to_f32(keys, dtype))
    limit = block_table.shape[1] * page_size
    for i in range(len(seq_ids)):
        b, p = int(seq_ids[i]), int(positions[i])
        if b < 0 or b >= block_table.shape[0] or p < 0 or p >= limit:
            continue
        page = int(block_table[b, p // page_size])
        cache[page, p % page_size] = codes[i]
        scales[page, p % page_size] = sc[i]
    return cache, scales

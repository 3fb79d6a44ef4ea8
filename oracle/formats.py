"""Decoding of stored indexer inputs to fp64 (oracle side; test infrastructure).

The pages say the indexer keys live in an FP8 cache (Lightning Indexer
explained, section 5 "Indexer-Cache"; Study MLA Indexer, data-flow diagram:
the key compressor ends in an FP8 quantisation).  They do not name the FP8
flavour; the reading taken here is OCP FP8 E4M3FN: 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no infinities,
and S.1111.111 as NaN (largest finite magnitude 448).  Each code is
multiplied by its fp32 scale.

bf16 is the upper half of an IEEE binary32 pattern: 1 sign bit, 8 exponent
bits with bias 127, 7 mantissa bits.

Everything is decoded from the bit fields with fp64 arithmetic, which is
exact for every finite code of both formats.
"""
from __future__ import annotations

import numpy as np


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes (uint8) -> fp64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** (1 - 7)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    m = (b & 0x7F).astype(np.float64)
    normal = (1.0 + m / 128.0) * np.exp2(e.astype(np.float64) - 127.0)
    sub = (m / 128.0) * 2.0 ** (1 - 127)
    v = np.where(e == 0, sub, normal)
    v = np.where(e == 255, np.where(m == 0, np.inf, np.nan), v)
    return sign * v


def decode(x: np.ndarray, dtype: str, scale: np.ndarray | None = None) -> np.ndarray:
    """Stored array -> fp64 values.

    dtype "f32": x is float32.  "bf16": x is uint16 bit patterns.
    "fp8": x is uint8 E4M3FN codes and ``scale`` (x.shape[:-1], fp32) is the
    per-row factor each decoded code is multiplied by.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "fp8":
        if scale is None:
            raise ValueError("fp8 input needs its per-row scale")
        return fp8_e4m3_to_f64(x) * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    raise ValueError(f"unknown dtype {dtype!r}")

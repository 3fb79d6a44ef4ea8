"""Pins of the K-cache write-path oracle (oracle/kcache.py) against the E4M3FN
format's own values, closed forms, brute force and invariants -- not against
its own formulas retyped."""
import numpy as np
import pytest

from oracle.formats import fp8_e4m3_to_f64
from oracle.kcache import encode_e4m3, kcache_append, key_rows_to_f32, quantize_keys



def test_encode_closed_form_codes():
    # values of the format: 1.0 = 0.0111.000, 448 = 0.1111.110 (largest finite),
    # 2^-9 = smallest subnormal, 2^-6 = smallest normal, 1.5 = 0.0111.100
    cases = [(0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -9, 0x01),
             (2.0 ** -6, 0x08), (1.5, 0x3C), (-1.5, 0xBC), (0.875 * 2.0 ** -6, 0x07), (240.0, 0x77)]
    for v, c in cases:
        assert int(encode_e4m3(np.array([v]))[0]) == c, (v, hex(c))


def test_encode_saturates_and_ties_to_even():
    # beyond the largest finite value: saturate (E4M3FN has no infinity)
    assert list(encode_e4m3(np.array([449.0, 500.0, 1e30, -1e30]))) == [0x7E, 0x7E, 0x7E, 0xFE]
    # exact midpoints go to the code whose mantissa ends in 0
    ties = {1.0625: 0x38,            # between 1.0 (0x38) and 1.125 (0x39)
            1.1875: 0x3A,            # between 1.125 (0x39) and 1.25 (0x3A)
            2.0 ** -10: 0x00,        # between 0 and 2^-9
            3 * 2.0 ** -10: 0x02,    # between 2^-9 (0x01) and 2^-8 (0x02)
            432.0: 0x7E,             # between 416 (0x7D) and 448 (0x7E)
            -1.0625: 0xB8}
    for v, c in ties.items():
        assert int(encode_e4m3(np.array([v]))[0]) == c, (v, hex(c))
    # just off a midpoint: plain nearest
    assert int(encode_e4m3(np.array([np.nextafter(1.0625, 2.0)]))[0]) == 0x39
    assert int(encode_e4m3(np.array([np.nextafter(1.1875, 0.0)]))[0]) == 0x39


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(encode_e4m3(fp8_e4m3_to_f64(codes)), codes)


def test_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.uniform(-460, 460, 20000), rng.normal(0, 0.01, 20000),
                        rng.normal(0, 2.0 ** -8, 5000)])
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = fp8_e4m3_to_f64(codes)
    got = encode_e4m3(y)
    mag = np.minimum(np.abs(y), 448.0) * np.where(np.signbit(y), -1.0, 1.0)
    dist = np.abs(mag[:, None] - vals[None, :])
    best = dist.min(axis=1)
    # the chosen code is among the nearest values, and the only one unless y is a midpoint
    got_dist = np.abs(mag - fp8_e4m3_to_f64(got))
    assert np.array_equal(got_dist, best)
    unique = (dist == best[:, None]).sum(axis=1) == 1
    assert np.array_equal(got[unique], codes[np.argmin(dist, axis=1)][unique])


def test_quantize_scale_and_error_bound():
    rng = np.random.default_rng(11)
    x = (rng.normal(size=(500, 128)) * np.exp(rng.uniform(-6, 6, size=(500, 1)))).astype(np.float32)
    codes, scale = quantize_keys(x)
    assert scale.dtype == np.float32
    amax = np.abs(x).max(axis=1)
    # the scale is absmax / 448 to fp32 rounding, and the absmax element gets the top code
    assert np.all(np.abs(scale.astype(np.float64) * 448.0 / amax - 1.0) < 2.0 ** -23)
    top = codes[np.arange(500), np.abs(x).argmax(axis=1)]
    assert np.all((top & 0x7F) == 0x7E)
    # every element within half a code step: relative 2^-4 for normals, 2^-10 absolute below
    back = fp8_e4m3_to_f64(codes) * scale[:, None].astype(np.float64)
    y = x.astype(np.float64) / scale[:, None]
    half_step = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * scale[:, None]
    assert np.all(np.abs(back - x) <= half_step * (1 + 1e-6))


def test_quantize_special_rows():
    codes, scale = quantize_keys(np.zeros((1, 128), np.float32))
    assert scale[0] == 1.0 and not codes.any()
    row = np.zeros(128, np.float32)
    row[0], row[1], row[2] = 448.0, -1.0, 0.5     # absmax 448: scale exactly 1, codes are the plain encodings
    codes, scale = quantize_keys(row[None])
    assert scale[0] == 1.0
    assert list(codes[0, :3]) == [0x7E, 0xB8, 0x30]
    codes, scale = quantize_keys(np.full((1, 128), -896.0, np.float32))
    assert scale[0] == 2.0 and np.all(codes == 0xFE)


def test_bf16_keys_widen_exactly():
    bits = np.array([0x3F80, 0xBFC0, 0x0000, 0x8000, 0x4380], np.uint16)   # 1, -1.5, 0, -0, 256
    f = key_rows_to_f32(bits, "bf16")
    assert list(f) == [1.0, -1.5, 0.0, -0.0, 256.0] and np.signbit(f[3])


def test_append_places_rows_by_block_table():
    page, D = 64, 128
    cache = np.full((6, page, D), 0x11, np.uint8)
    scales = np.full((6, page), -1.0, np.float32)
    table = np.array([[4, 1, 5], [0, 2, 3]], np.int32)
    rng = np.random.default_rng(3)
    keys = rng.normal(size=(6, D)).astype(np.float32)
    seq = np.array([0, 0, 1, -1, 1, 0], np.int32)
    pos = np.array([0, 130, 64, 5, 192, 63], np.int32)   # (1, 192) is past 3 pages: dropped; -1: padding
    new_cache, new_scales = kcache_append(cache, scales, keys, "f32", seq, pos, table, page)
    codes, sc = quantize_keys(keys)
    assert np.array_equal(new_cache[4, 0], codes[0]) and new_scales[4, 0] == sc[0]
    assert np.array_equal(new_cache[5, 2], codes[1]) and new_scales[5, 2] == sc[1]
    assert np.array_equal(new_cache[2, 0], codes[2]) and new_scales[2, 0] == sc[2]
    assert np.array_equal(new_cache[4, 63], codes[5]) and new_scales[4, 63] == sc[5]
    written = np.zeros((6, page), bool)
    written[4, 0] = written[5, 2] = written[2, 0] = written[4, 63] = True
    assert np.all(new_cache[~written] == 0x11) and np.all(new_scales[~written] == -1.0)
    assert np.all(cache == 0x11)  # inputs untouched

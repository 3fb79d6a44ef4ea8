"""Pins of the oracle's input decoding against torch's own dtype casts and
closed-form code values (CPU only)."""
import math

import numpy as np
import torch

from oracle import brute, formats


def test_fp8_all_codes_match_torch_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero is kept
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_fp8_closed_form_codes():
    v = formats.fp8_e4m3_to_f64(np.array([0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE, 0x40, 0x00], np.uint8))
    assert v[0] == 2.0 ** -9          # smallest subnormal
    assert v[1] == 7 * 2.0 ** -9      # largest subnormal
    assert v[2] == 2.0 ** -6          # smallest normal
    assert v[3] == 1.0
    assert v[4] == 448.0              # largest finite (no infinities in E4M3FN)
    assert v[5] == -448.0
    assert v[6] == 2.0
    assert v[7] == 0.0


def test_fp8_scalar_twin_matches_vectorised():
    codes = np.arange(256, dtype=np.uint8)
    vec = formats.fp8_e4m3_to_f64(codes)
    for c in range(256):
        s = brute.fp8_value(c)
        if math.isnan(vec[c]):
            assert math.isnan(s)
        else:
            assert s == vec[c]


def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = formats.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    for b in (0x0000, 0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x8000):
        assert brute.bf16_value(b) == ours[b]


def test_fp8_scale_is_applied_per_row():
    codes = np.array([[0x38, 0x40], [0x38, 0xB8]], np.uint8)
    scale = np.array([0.5, 3.0], np.float32)
    v = formats.decode(codes, "fp8", scale)
    assert v.tolist() == [[0.5, 1.0], [3.0, -3.0]]

"""The seeded generators: determinism, byte formats and workload structure (CPU)."""
import numpy as np

import synth
from oracle import formats


def test_same_seed_same_bytes():
    a = synth.prefill_inputs(1, 64, 4, 32, "fp8", 9)
    b = synth.prefill_inputs(1, 64, 4, 32, "fp8", 9)
    for key in ("q", "q_scale", "k", "k_scale", "w"):
        assert np.array_equal(a[key], b[key])
    c = synth.prefill_inputs(1, 64, 4, 32, "fp8", 10)
    assert not np.array_equal(a["q"], c["q"])


def test_fp8_quantiser_is_saturating_nearest():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((500, 128)).astype(np.float32) * rng.uniform(0.01, 100, (500, 1)).astype(np.float32)
    x[3] = 0.0
    codes, scale = synth.quantize_fp8_rows(x)
    assert scale[3] == 1.0
    assert not np.any((codes & 0x7F) == 0x7F)                     # never NaN
    v = formats.fp8_e4m3_to_f64(codes)
    y = x.astype(np.float64) / scale.astype(np.float64)[:, None]
    assert np.all(np.abs(v).max(axis=1)[np.arange(500) != 3] == 448.0)  # absmax hits 448
    # nearest: no other finite code is closer than the chosen one
    table = formats.fp8_e4m3_to_f64(np.arange(256, dtype=np.uint8))
    finite = table[np.isfinite(table)]
    sub = rng.choice(y.size, 2000, replace=False)
    for yy, vv in zip(y.reshape(-1)[sub], v.reshape(-1)[sub]):
        assert abs(vv - yy) <= np.min(np.abs(finite - yy)) * (1 + 1e-12) + 1e-300


def test_bf16_is_round_to_nearest():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10000).astype(np.float32)
    v = formats.bf16_to_f64(synth.to_bf16_bits(x))
    assert np.all(np.abs(v - x) <= np.abs(x) * 2.0 ** -8)


def test_weights_are_softmax_rows():
    d = synth.prefill_inputs(1, 32, 64, 16, "f32", 3)
    s = d["w"].astype(np.float64).sum(-1)
    assert np.allclose(s, 1.0, atol=1e-6) and np.all(d["w"] > 0)


def test_needles_planted_per_block():
    d = synth.prefill_inputs(1, 256, 8, 16, "bf16", 2, needles=True)
    pos = [p for (_, _, p) in d["needles"]]
    assert len(pos) == 4 and all(len(p) == 32 for p in pos)
    allp = np.concatenate(pos)
    assert len(set(allp.tolist())) == allp.size          # distinct across blocks
    for j, p in enumerate(pos):
        assert p.max() < (j + 1) * 64                       # inside [0, block_end)


def test_paged_decode_layout():
    d = synth.decode_inputs(5, (10, 300), 4, 32, seed=5, page_size=64, permute=True, extra_pages=3)
    ctx = d["context_lens"]
    assert np.all((ctx >= 10) & (ctx <= 300))
    used = []
    for b in range(5):
        n = -(-int(ctx[b]) // 64)
        used += d["block_table"][b, :n].tolist()
    assert len(set(used)) == len(used) == d["num_pages"] - 3
    assert d["k_cache"].shape == (d["num_pages"], 64, 32)
    d2 = synth.decode_inputs(2, [128, 128], 4, 32, seed=5, permute=False)
    assert d2["block_table"].tolist() == [[0, 1], [2, 3]]

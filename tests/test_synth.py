"""The seeded input generator: determinism, shapes, and the value
distributions the workloads call for.  CPU only."""
import json
import os

import numpy as np

import synth


def test_deterministic():
    a = synth.make_random(2, 256, 16, 5, outlier_frac=0.01)
    b = synth.make_random(2, 256, 16, 5, outlier_frac=0.01)
    for u, v in ((a.x, b.x), (a.weights.W, b.weights.W), (a.weights.scale, b.weights.scale),
                 (a.weights.mn, b.weights.mn)):
        assert np.array_equal(u, v)
    c = synth.make_random(2, 256, 16, 6)
    assert not np.array_equal(a.weights.W, c.weights.W)


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 lies exactly between bf16 neighbours 1 and 1 + 2^-7 -> even (1).
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.0, 0.0], dtype=np.float64)
    bits = synth.to_bf16_bits(vals)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000]
    assert np.array_equal(synth.bf16_bits_to_f32(bits), np.array([1, 1, 1 + 2 ** -6, -2, 0], np.float32))


def test_distributions():
    rng = synth.rng_for(0)
    wt = synth.draw_weights(rng, 1024, 512)
    assert wt.W.shape == (512, 128) and wt.scale.shape == (512, 8) and wt.mn.shape == (512, 8)
    nib = np.stack([(wt.W >> (4 * i)) & 0xF for i in range(8)]).ravel()
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * nib.size / 16 and counts.max() < 1.1 * nib.size / 16
    s = synth.bf16_bits_to_f32(wt.scale).astype(np.float64)
    m = synth.bf16_bits_to_f32(wt.mn).astype(np.float64)
    assert s.min() >= 1e-4 * 0.99 and abs(np.median(s) - (0.01 * 0.6745 + 1e-4)) < 1e-3
    assert np.std(m + 8 * s) < 1.2e-3 and abs(np.mean(m + 8 * s)) < 2e-4


def test_outliers_per_row():
    K = 17408
    rng = synth.rng_for(3)
    x = synth.draw_x(rng, 2, K, outlier_frac=0.01)
    v = np.abs(synth.bf16_bits_to_f32(x))
    assert x.shape == (2, K)
    # 174 entries per row were scaled by 20; |20 z| > 5 for about 80% of them,
    # while N(0,1) alone essentially never exceeds 5.
    for row in v:
        assert 100 < int((row > 5).sum()) <= 174
    v0 = np.abs(synth.bf16_bits_to_f32(synth.draw_x(synth.rng_for(3), 2, K)))
    assert int((v0 > 5).sum()) < 3


def test_workloads_and_stream_bytes():
    w = synth.WORKLOADS
    assert (w["gateup"].K, w["gateup"].N) == (5120, 34816)
    assert (w["down"].K, w["down"].N) == (17408, 5120)
    assert w["verify"].M == 7
    per_layer = sum(synth.algorithmic_bytes(1, K, N) for K, N in synth.STREAM_LAYER_SHAPES)
    head = synth.algorithmic_bytes(1, *synth.STREAM_HEAD_SHAPE)
    assert per_layer == 192481280 and head == 357050368
    assert 64 * per_layer + head == 12675852288


def test_byte_accounting_matches_format():
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
    f = fx["format"]
    bits = f["code_bits"] + (f["scale_bits"] + f["min_bits"]) / f["group"]
    assert bits == f["bits_per_weight"]
    K, N = 5120, 34816
    weight_bytes = synth.algorithmic_bytes(1, K, N) - 2 * K - 4 * N
    assert weight_bytes * 8 == f["bits_per_weight"] * K * N
    b = fx["bandwidth"]
    assert round(b["read_GBps"] / b["weight_GB"]) == b["ceiling_tok_s"]


def test_verify_rows_shared_across_M():
    c8 = synth.make_case("verify", 8)
    c3 = synth.make_case("verify", 3)
    assert np.array_equal(c8.x[:3], c3.x) and np.array_equal(c8.weights.W, c3.weights.W)

"""Pins that tie the oracle's quantizer (bf16 weights -> int4-g128 codes,
scale, minimum) to facts outside itself.

Each ``qpin_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` when
the quantizer disagrees with the fact:
  * a group lying exactly on a grid of 16 bf16 levels is recovered exactly,
    by round-to-nearest and by the range search (its first candidate already
    has zero error);
  * a group worked by hand (codes, scale, minimum and error in closed form);
  * a constant group gets code 0, scale 0 and the constant as minimum;
  * every code is the nearest of the 16 levels of its group's scale and
    minimum, or 0 / 15 for weights below / above the levels;
  * the reported squared error equals the error of dequantizing the output
    with the oracle's (separately pinned) dequant;
  * the range search is never worse than round-to-nearest, and on a group
    with one far outlier it is strictly better and gives the outlier code 15.
"""
from __future__ import annotations

import numpy as np

import synth


def _bits(values):
    return synth.to_bf16_bits(np.asarray(values, dtype=np.float32))


def _values(bits):
    return synth.bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def qpin_grid_exact(orc):
    """v = (q - 8) * 2^-6 for codes q covering 0..15: scale 2^-6, minimum
    -2^-3, the codes themselves, error 0."""
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(3, 256))
    q[:, 0], q[:, 1], q[:, 128], q[:, 129] = 0, 15, 15, 0      # every group spans the full range
    w = _bits((q - 8) * 2.0 ** -6)
    for ncand in (1, 9):
        W, S, Mn, err = orc.quantize(w, ncand)
        assert np.array_equal(orc.codes(W), q), ncand
        assert np.all(_values(S) == 2.0 ** -6) and np.all(_values(Mn) == -2.0 ** -3), ncand
        assert np.all(err == 0.0), ncand


def qpin_worked_rtn(orc):
    """Worked by hand: v_0 = 0, v_1 = 15/16 and, for k >= 2, v_k = j/16 + 1/64
    (k even) or j/16 - 1/64 (k odd) with j = 1 + k mod 14, all exact in bf16.
    The range is [0, 15/16], so round-to-nearest has scale 1/16 and minimum
    0; (v_k - 0)/(1/16) = j +- 1/4 rounds to code j; v_0, v_1 get codes 0 and
    15 exactly, and every other weight is off by 1/64: error 126/4096."""
    k = np.arange(128)
    j = 1 + k % 14
    v = j / 16.0 + np.where(k % 2 == 0, 1.0, -1.0) / 64.0
    v[0], v[1] = 0.0, 15.0 / 16.0
    q = j.copy()
    q[0], q[1] = 0, 15
    W, S, Mn, err = orc.quantize(_bits(v[None, :]), 1)
    assert np.array_equal(orc.codes(W)[0], q)
    assert _values(S)[0, 0] == 1.0 / 16.0 and _values(Mn)[0, 0] == 0.0
    assert err[0, 0] == 126.0 / 4096.0


def qpin_constant_group(orc):
    """A constant group: code 0 everywhere, scale 0, minimum = the constant."""
    w = np.concatenate([_bits(np.full((2, 128), 0.375)), _bits(np.zeros((2, 128)))], axis=1)
    W, S, Mn, err = orc.quantize(w, 9)
    assert np.all(orc.codes(W) == 0)
    assert np.all(_values(S) == 0.0)
    assert np.array_equal(_values(Mn), np.array([[0.375, 0.0], [0.375, 0.0]]))
    assert np.all(err == 0.0)


def _random_weights(seed, N=6, K=512):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    w[:, 7] *= 25.0                                   # an outlier in the first group of every row
    return _bits(w)


def qpin_nearest_level(orc):
    """Each code is the nearest level q*s + m (|v - level| <= s/2), or the end
    code for weights outside the 16 levels."""
    for ncand in (1, 9):
        w = _random_weights(11 + ncand)
        W, S, Mn, _ = orc.quantize(w, ncand)
        q = orc.codes(W).astype(np.float64)
        v = _values(w)
        N, K = v.shape
        s = np.repeat(_values(S), 128, axis=1)
        m = np.repeat(_values(Mn), 128, axis=1)
        level = q * s + m
        inside = (v >= m - s / 2) & (v <= m + 15 * s + s / 2)
        assert np.all(np.abs(v - level)[inside] <= s[inside] / 2 * (1 + 1e-12)), ncand
        assert np.all(q[v < m - s / 2] == 0) and np.all(q[v > m + 15 * s + s / 2] == 15), ncand


def qpin_error_is_dequant_error(orc):
    """The reported error is the squared distance of the dequantized weights."""
    w = _random_weights(21)
    W, S, Mn, err = orc.quantize(w, 9)
    rec = orc.dequant_f64(W, S, Mn)
    d2 = ((rec - _values(w)) ** 2).reshape(w.shape[0], -1, 128).sum(axis=2)
    assert np.allclose(d2, err, rtol=1e-12, atol=0.0)


def qpin_search_beats_round_to_nearest(orc):
    """The range search never loses to round-to-nearest; on groups holding
    one outlier 25 times the others' spread, clipping wins on most, and an
    outlier near a tight cluster is clipped to code 15."""
    w = _random_weights(31)
    err1 = orc.quantize(w, 1)[3]
    err9 = orc.quantize(w, 9)[3]
    assert np.all(err9 <= err1)
    assert np.mean(err9[:, 0] < err1[:, 0]) >= 0.5          # the groups with the outlier
    g = np.zeros((1, 128), dtype=np.float32)
    g[0, :127] = np.linspace(-1.0, 1.0, 127)
    g[0, 127] = 1.3
    gb = _bits(g)
    e1 = orc.quantize(gb, 1)[3]
    Wg, Sg, Mg, e9 = orc.quantize(gb, 9)
    assert e9[0, 0] < e1[0, 0]
    assert orc.codes(Wg)[0, 127] == 15 and _values(Mg)[0, 0] + 15 * _values(Sg)[0, 0] < 1.3


ALL_QPINS = [qpin_worked_rtn, qpin_grid_exact, qpin_constant_group, qpin_nearest_level, qpin_error_is_dequant_error,
             qpin_search_beats_round_to_nearest]

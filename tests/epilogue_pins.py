"""Pins that tie the oracle's epilogues (SwiGLU on a fused gate/up product;
residual add + RMSNorm) to facts outside the oracle.

Each ``epin_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` when
the epilogue disagrees with the fact:
  * silu(g) - silu(-g) = g and silu(g) + silu(-g) = g tanh(g/2) for every g
    (the logistic function's symmetry; tanh from the maths library);
  * worked values: silu(ln 3) = (3/4) ln 3, silu(0) = 0, silu of a large
    positive g is g and of a large negative g is 0 to within e^-|g| |g|;
  * the gate half is the first half of the fused columns;
  * RMSNorm worked by hand: h = (3, 4, 0, 0) has mean square 25/4, so with
    eps = 0 the output is h / 2.5 * gamma, and with eps = 2.75 it is h / 3;
  * with eps = 0, scaling r and y by a power of two leaves the output
    unchanged bit for bit, and the output has mean square 1 for gamma = 1;
  * a zero row stays zero for eps > 0, and a row of ones with eps = 3 is
    halved;
  * each row is normalised on its own.
"""
from __future__ import annotations

import math

import numpy as np

import synth


def _ulps(a, b):
    return np.abs(a - b) / np.spacing(np.maximum(np.abs(a), np.abs(b)) + 1e-300)


def epin_silu_odd_identity(orc):
    g = np.concatenate([np.linspace(-30.0, 30.0, 241), [1e-3, 0.7, 2.5, 17.0]])
    I = 2 * g.size
    y = np.concatenate([np.concatenate([g, -g]), np.ones(I)])[None, :]
    act = orc.swiglu(y)[0]
    d = act[:g.size] - act[g.size:]
    assert np.all(np.abs(d - g) <= 4 * np.spacing(np.abs(g)) + 4 * np.spacing(np.abs(act[:g.size]))), \
        np.max(np.abs(d - g))
    s = act[:g.size] + act[g.size:]
    even = g * np.tanh(g / 2.0)
    assert np.all(np.abs(s - even) <= 1e-14 * np.abs(g) + 1e-300), np.max(np.abs(s - even))


def epin_swiglu_worked(orc):
    big = 50.0
    y = np.array([[math.log(3.0), 0.0, big, -big, 2.0, 7.0, 3.0, 5.0]])
    act = orc.swiglu(y)[0]
    assert _ulps(act[0], 1.5 * math.log(3.0)) <= 4, act[0]
    assert act[1] == 0.0
    assert abs(act[2] - 3.0 * big) <= 3.0 * big * 1e-20 + np.spacing(3.0 * big) * 2
    assert abs(act[3]) <= 5.0 * big * math.exp(-big) * 1.01


def epin_rmsnorm_worked(orc):
    r = np.array([[1.0, 2.0, 0.0, 0.0]])
    y = np.array([[2.0, 2.0, 0.0, 0.0]])
    gamma = synth.to_bf16_bits(np.array([1.0, 0.5, 2.0, 1.0]))
    h, out = orc.residual_rmsnorm(y, r, gamma, 0.0)
    assert np.array_equal(h, [[3.0, 4.0, 0.0, 0.0]])
    assert np.all(_ulps(out[0], np.array([1.2, 0.8, 0.0, 0.0])) <= 4), out
    _, out = orc.residual_rmsnorm(y, r, synth.to_bf16_bits(np.ones(4)), 2.75)    # mean square + eps = 9
    assert np.all(_ulps(out[0], np.array([1.0, 4.0 / 3.0, 0.0, 0.0])) <= 4), out


def epin_rmsnorm_invariants(orc):
    rng = np.random.default_rng(71)
    N = 300
    r = rng.standard_normal((2, N))
    y = rng.standard_normal((2, N)) * 3.0
    gamma = synth.to_bf16_bits(rng.standard_normal(N))
    _, out = orc.residual_rmsnorm(y, r, gamma, 0.0)
    for j in (-7, 3):
        _, out2 = orc.residual_rmsnorm(y * 2.0 ** j, r * 2.0 ** j, gamma, 0.0)
        assert np.array_equal(out, out2), j
    _, out1 = orc.residual_rmsnorm(y, r, synth.to_bf16_bits(np.ones(N)), 0.0)
    assert np.all(np.abs(np.mean(out1 ** 2, axis=1) - 1.0) <= 1e-13)
    ones = synth.to_bf16_bits(np.ones(N))
    z = np.zeros((1, N))
    _, o0 = orc.residual_rmsnorm(z, z, ones, 1e-6)                # a zero row stays zero when eps > 0
    assert np.all(o0 == 0.0)
    _, oc = orc.residual_rmsnorm(np.ones((1, N)), z, ones, 3.0)   # mean square 1, + eps = 4: halved
    assert np.all(oc == 0.5)
    for m in range(2):                                            # rows on their own
        _, om = orc.residual_rmsnorm(y[m:m + 1], r[m:m + 1], gamma, 1e-6)
        _, oall = orc.residual_rmsnorm(y, r, gamma, 1e-6)
        assert np.array_equal(om[0], oall[m])


ALL_EPINS = [epin_silu_odd_identity, epin_swiglu_worked, epin_rmsnorm_worked, epin_rmsnorm_invariants]

"""Pins that tie the fp64 oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` when the
oracle disagrees with the fact.  ``test_oracle.py`` runs them against the real
oracle; ``test_oracle_mutants.py`` runs them against copies built with one
planted mistake each and checks that every mistake trips at least one pin.

What they pin against, none of it the oracle's own code:
  * hand-worked fixtures under tests/golden/ (nibble order, bf16 values,
    two small products worked out by hand);
  * exact rational brute force (fractions.Fraction) on tiny random shapes,
    with its own bf16 decoder written from the bit-field definition;
  * closed forms for constant codes, one-hot activations and all-ones rows;
  * linearity (disjoint-support split, exact power-of-two scaling) and the
    row independence of an M-row product.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- independent exact helpers (rational arithmetic, written from definitions)

def bf16_exact(bits: int) -> Fraction:
    """bf16 value from its fields: sign, 8-bit biased exponent, 7-bit fraction."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    assert e != 0xFF, "non-finite bf16"
    if e == 0:
        mag = Fraction(f, 128) * Fraction(1, 2 ** 126)
    else:
        mag = Fraction(128 + f, 128) * (Fraction(2) ** (e - 127))
    return sign * mag


def nibbles_of_word(word: int):
    """Hex digits of the word, least significant first."""
    return [int(c, 16) for c in reversed(f"{word:08x}")]


def exact_product(x, W, scale, mn):
    """Exact rational y and a for uint16 x [M][K], uint32 W [N][K/8]."""
    M, K = x.shape
    N = W.shape[0]
    codes = [[d for word in W[n] for d in nibbles_of_word(int(word))] for n in range(N)]
    y = [[Fraction(0)] * N for _ in range(M)]
    a = [[Fraction(0)] * N for _ in range(M)]
    xs = [[bf16_exact(int(v)) for v in row] for row in x]
    for n in range(N):
        wcol = [codes[n][k] * bf16_exact(int(scale[n][k // 128])) + bf16_exact(int(mn[n][k // 128]))
                for k in range(K)]
        for m in range(M):
            tot = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                p = xs[m][k] * wcol[k]
                tot += p
                mag += abs(p)
            y[m][n] = tot
            a[m][n] = mag
    return y, a


def _words_from_fixture(cols, K):
    per = K // 8
    out = []
    for words in cols:
        ws = [int(w, 16) for w in words]
        out.append([ws[j % len(ws)] for j in range(per)])
    return np.array(out, dtype=np.uint32)


def _x_from_fixture(rows, K):
    x = np.zeros((len(rows), K), dtype=np.uint16)
    for m, spec in enumerate(rows):
        for i in range(0, len(spec), 2):
            val, where = int(spec[i], 16), spec[i + 1]
            if where == "all":
                x[m, :] = val
            elif where == "k<128":
                x[m, :128] = val
            elif where == "k>=128":
                x[m, 128:] = val
            else:
                raise ValueError(where)
    return x


def _hex_grid(rows):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=np.uint16)


# --- pins ---------------------------------------------------------------------

def pin_nibble_order(orc):
    fx = golden("nibble_order.json")
    for case in fx["cases"]:
        W = np.array([[int(case["word"], 16)] * 16], dtype=np.uint32)   # K = 128
        q = orc.codes(W)
        assert list(q[0, :8]) == case["codes"], (case, list(q[0, :8]))
        assert list(q[0, 8:16]) == case["codes"], case


def pin_bf16_values(orc):
    """Code 0 leaves the minimum, code 1 with minimum 0 leaves the scale."""
    fx = golden("bf16_values.json")
    bits = [int(c["bits"], 16) for c in fx["cases"]]
    vals = [Fraction(c["value"]) for c in fx["cases"]]
    n = len(bits)
    zero_codes = np.zeros((n, 16), dtype=np.uint32)
    one_codes = np.full((n, 16), 0x11111111, dtype=np.uint32)
    bf = np.array(bits, dtype=np.uint16).reshape(n, 1)
    z = np.zeros((n, 1), dtype=np.uint16)
    w_min = orc.dequant_f64(zero_codes, z + 0x3F80, bf)
    w_scale = orc.dequant_f64(one_codes, bf, z)
    for i in range(n):
        assert Fraction(w_min[i, 0]) == vals[i], (hex(bits[i]), w_min[i, 0], vals[i])
        assert Fraction(w_min[i, 127]) == vals[i]
        assert Fraction(w_scale[i, 77]) == vals[i], (hex(bits[i]), w_scale[i, 77])


def pin_worked_examples(orc):
    fx = golden("worked_examples.json")
    for ex in fx["examples"]:
        K = ex["K"]
        W = _words_from_fixture(ex["words"], K)
        scale = _hex_grid(ex["scale"])
        mn = _hex_grid(ex["min"])
        x = _x_from_fixture(ex["x"], K)
        y, a = orc.gemm(x, W, scale, mn)
        want_y = np.array([[float(Fraction(v)) for v in r] for r in ex["y"]])
        want_a = np.array([[float(Fraction(v)) for v in r] for r in ex["a"]])
        assert np.array_equal(y, want_y), (ex["name"], y, want_y)
        assert np.array_equal(a, want_a), (ex["name"], a, want_a)


def pin_bruteforce(orc, seeds=(11, 12, 13, 14)):
    """Exact rational sums on tiny random shapes.  The fp64 k-ascending sum
    must lie within K * 2^-53 * a of the exact value."""
    shapes = [(1, 128, 3), (2, 256, 5), (3, 128, 8), (3, 256, 2)]
    for seed, (M, K, N) in zip(seeds, shapes):
        case = synth.make_random(M, K, N, seed, outlier_frac=0.02)
        wt = case.weights
        y, a = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
        ye, ae = exact_product(case.x, wt.W, wt.scale, wt.mn)
        w64 = orc.dequant_f64(wt.W, wt.scale, wt.mn)
        for m in range(M):
            for n in range(N):
                bound = float(ae[m][n]) * K * 2.0 ** -53
                err = abs(Fraction(y[m, n]) - ye[m][n])
                assert err <= Fraction(bound), (seed, m, n, float(err), bound)
                assert abs(a[m, n] - float(ae[m][n])) <= bound + 1e-300
        codes = [[d for word in wt.W[n] for d in nibbles_of_word(int(word))] for n in range(N)]
        for n in range(N):
            for k in range(0, K, 7):
                we = codes[n][k] * bf16_exact(int(wt.scale[n][k // 128])) + bf16_exact(int(wt.mn[n][k // 128]))
                assert Fraction(w64[n, k]) == we, (seed, n, k)


def pin_constant_codes(orc):
    """q = c everywhere: y[m][n] = sum_g (c*s_g + m_g) * X_g, X_g = sum of x in
    group g.  With x = 1 and one scale/minimum, y = K*(c*s + m) exactly."""
    K, N = 384, 3
    s_bits, m_bits = 0x3E80, 0xBF00          # 1/4, -1/2
    for c in (0, 1, 7, 15):
        W = np.full((N, K // 8), int(f"{c:x}" * 8, 16), dtype=np.uint32)
        scale = np.full((N, K // 128), s_bits, dtype=np.uint16)
        mn = np.full((N, K // 128), m_bits, dtype=np.uint16)
        x = np.full((1, K), 0x3F80, dtype=np.uint16)
        y, a = orc.gemm(x, W, scale, mn)
        want = K * (c * Fraction(1, 4) - Fraction(1, 2))
        assert np.all(y == float(want)), (c, y, want)
        assert np.all(a == float(abs(want))), (c, a)
    rng = synth.rng_for(21)
    for c in (3, 12):
        G = 3
        W = np.full((N, G * 16), int(f"{c:x}" * 8, 16), dtype=np.uint32)
        scale = synth.to_bf16_bits(rng.uniform(0.01, 0.1, (N, G)))
        mn = synth.to_bf16_bits(rng.uniform(-1, 1, (N, G)))
        x = synth.to_bf16_bits(rng.standard_normal((2, G * 128)))
        y, a = orc.gemm(x, W, scale, mn)
        for m in range(2):
            for n in range(N):
                want = Fraction(0)
                for g in range(G):
                    Xg = sum(bf16_exact(int(v)) for v in x[m, g * 128:(g + 1) * 128])
                    want += (c * bf16_exact(int(scale[n, g])) + bf16_exact(int(mn[n, g]))) * Xg
                assert abs(Fraction(y[m, n]) - want) <= Fraction(a[m, n]) * G * 128 * Fraction(1, 2 ** 52)


def pin_one_hot(orc):
    """x = e_k picks out w[n][k] exactly; that value rounded once is w32."""
    case = synth.make_random(1, 512, 6, 31)
    wt = case.weights
    w64 = orc.dequant_f64(wt.W, wt.scale, wt.mn)
    w32 = orc.dequant_f32(wt.W, wt.scale, wt.mn)
    assert np.array_equal(w32, w64.astype(np.float32))
    for k in (0, 1, 7, 8, 127, 128, 200, 511):
        x = np.zeros((1, 512), dtype=np.uint16)
        x[0, k] = 0x3F80
        y, a = orc.gemm(x, wt.W, wt.scale, wt.mn)
        assert np.array_equal(y[0], w64[:, k]), k
        assert np.array_equal(a[0], np.abs(w64[:, k])), k


def pin_linearity(orc):
    """x = x1 + x2 with disjoint supports: y(x) = y(x1) + y(x2) up to rounding;
    y(2x) = 2 y(x) exactly (doubling a bf16 only moves its exponent)."""
    case = synth.make_random(3, 768, 7, 41)
    wt = case.weights
    x = case.x
    rng = synth.rng_for(42)
    mask = rng.random(x.shape) < 0.5
    x1 = np.where(mask, x, 0).astype(np.uint16)
    x2 = np.where(mask, 0, x).astype(np.uint16)
    y, a = orc.gemm(x, wt.W, wt.scale, wt.mn)
    y1, _ = orc.gemm(x1, wt.W, wt.scale, wt.mn)
    y2, _ = orc.gemm(x2, wt.W, wt.scale, wt.mn)
    assert np.all(np.abs(y - (y1 + y2)) <= 3 * 768 * 2.0 ** -53 * a)
    x2x = x.copy()
    nz = (x2x & 0x7F80) != 0
    x2x[nz] = x2x[nz] + 0x0080                 # exponent + 1 on normal values
    sub = ~nz & ((x2x & 0x7FFF) != 0)
    assert not sub.any()
    yd, ad = orc.gemm(x2x, wt.W, wt.scale, wt.mn)
    assert np.array_equal(yd, 2 * y) and np.array_equal(ad, 2 * a)


def pin_rows(orc):
    """Row m of an M-row product equals the one-row product of x[m], bit for
    bit (each output row depends on its own activation row only)."""
    case = synth.make_random(8, 640, 9, 51, outlier_frac=0.01)
    wt = case.weights
    y, a = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    for m in range(8):
        y1, a1 = orc.gemm(case.x[m:m + 1], wt.W, wt.scale, wt.mn)
        assert np.array_equal(y[m], y1[0]) and np.array_equal(a[m], a1[0]), m
    cols = np.array([8, 0, 3], dtype=np.int64)
    yc, ac = orc.gemm(case.x, wt.W, wt.scale, wt.mn, cols=cols)
    assert np.array_equal(yc, y[:, cols]) and np.array_equal(ac, a[:, cols])


ALL_PINS = [pin_nibble_order, pin_bf16_values, pin_worked_examples, pin_bruteforce,
            pin_constant_codes, pin_one_hot, pin_linearity, pin_rows]

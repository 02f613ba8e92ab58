"""Seeded synthetic inputs for the int4-g128 weight-streaming product.

This module is shared by the HIP path's tests and benchmark and by the oracle's
tests.  It only draws and encodes inputs; it holds none of the product's
arithmetic (no unpacking, no dequantisation, no products).

Distributions stand in for the quantised checkpoint matrices and decode
activations that the Token Rush README measures on (its quality table and
bandwidth paragraph), which are not available here:

* codes: every nibble uniform on 0..15.  Drawing each packed uint32 word
  uniformly on [0, 2^32) gives exactly that, with no packing arithmetic;
* scale: bf16(|N(0,1)| * 0.01 + 1e-4), one per (column, 128-group);
* minimum: bf16(-8 * scale + N(0, sd=1e-3)), using the already rounded scale,
  so the minimum sits near the value a centred code of 8 would cancel;
* x: bf16(N(0,1)), optionally with round(0.01*K) distinct positions per row
  (chosen uniformly without replacement) multiplied by 20 before rounding, the
  activation outliers of the down projection.

Draw order from one ``numpy.random.Generator(PCG64(seed))``: codes, scale,
minimum noise, x.  Real values are formed in float64, rounded to float32, then
rounded to bf16 (nearest, ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 128


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(values) -> np.ndarray:
    """float64/float32 array -> bf16 bit patterns (uint16), via float32,
    round to nearest even on the dropped 16 bits (finite inputs only)."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Weights:
    W: np.ndarray       # uint32 [N][K/8]
    scale: np.ndarray   # uint16 (bf16 bits) [N][K/128]
    mn: np.ndarray      # uint16 (bf16 bits) [N][K/128]

    @property
    def N(self) -> int:
        return self.W.shape[0]

    @property
    def K(self) -> int:
        return 8 * self.W.shape[1]


def draw_weights(rng: np.random.Generator, K: int, N: int) -> Weights:
    if K % GROUP or K <= 0 or N <= 0:
        raise ValueError(f"K must be a positive multiple of {GROUP} and N positive (K={K}, N={N})")
    G = K // GROUP
    W = rng.integers(0, 1 << 32, size=(N, K // 8), dtype=np.uint32)
    scale = to_bf16_bits(np.abs(rng.standard_normal((N, G))) * 0.01 + 1e-4)
    noise = rng.standard_normal((N, G)) * 1e-3
    mn = to_bf16_bits(-8.0 * bf16_bits_to_f32(scale).astype(np.float64) + noise)
    return Weights(W, scale, mn)


def draw_dense_weights(rng: np.random.Generator, N: int, K: int, sigma: float = 0.02,
                       outlier_frac: float = 1e-3, outlier_gain: float = 25.0) -> np.ndarray:
    """Unquantized weights as bf16 bits [N][K] (row n = the K weights of
    output column n): N(0, sigma^2), with round(outlier_frac * N * K) entries
    chosen uniformly without replacement multiplied by outlier_gain."""
    w = rng.standard_normal((N, K)) * sigma
    n_out = int(round(outlier_frac * N * K))
    if n_out:
        idx = rng.choice(N * K, size=n_out, replace=False)
        w.reshape(-1)[idx] *= outlier_gain
    return to_bf16_bits(w)


def draw_x(rng: np.random.Generator, M: int, K: int, outlier_frac: float = 0.0,
           outlier_gain: float = 20.0) -> np.ndarray:
    x = rng.standard_normal((M, K))
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * K))
        for m in range(M):
            idx = rng.choice(K, size=n_out, replace=False)
            x[m, idx] *= outlier_gain
    return to_bf16_bits(x)


@dataclass
class Case:
    name: str
    M: int
    K: int
    N: int
    weights: Weights
    x: np.ndarray       # uint16 (bf16 bits) [M][K]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    seed: int
    outlier_frac: float = 0.0
    description: str = ""


# The single-matrix workloads.  N = 34816 is two 17408-wide projections fused
# side by side (rows 0..17407 and 17408..34815); the product treats it as one N.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1024, 1024, 0, 0.0, "tiny GEMV, M=1 K=1024 N=1024"),
    "gateup": Workload("gateup", 1, 5120, 34816, 1, 0.0,
                       "decode gate/up projection, M=1 K=5120 N=34816"),
    "down": Workload("down", 1, 17408, 5120, 2, 0.01,
                     "decode down projection with 1% activation outliers x20, M=1 K=17408 N=5120"),
    "verify": Workload("verify", 7, 5120, 34816, 3, 0.0,
                       "speculative verify, M=7 K=5120 N=34816 (swept M=1..8 on the first M of 8 rows)"),
}

# Whole decode-step weight stream: 64 layers x four matrices plus an output
# projection, one seed per distinct shape (4 + shape index).
STREAM_LAYER_SHAPES = [(5120, 12288), (6144, 5120), (5120, 34816), (17408, 5120)]
STREAM_HEAD_SHAPE = (5120, 131072)
STREAM_LAYERS = 64


def stream_shapes():
    """Distinct (K, N, seed) of the decode-step stream, in launch order."""
    shapes = [(K, N, 4 + i) for i, (K, N) in enumerate(STREAM_LAYER_SHAPES)]
    shapes.append((STREAM_HEAD_SHAPE[0], STREAM_HEAD_SHAPE[1], 4 + len(STREAM_LAYER_SHAPES)))
    return shapes


def make_case(name: str, M: int | None = None) -> Case:
    """Draw a named workload.  ``verify`` always draws 8 rows and keeps the
    first M, so row m holds the same data for every M of the sweep."""
    w = WORKLOADS[name]
    rng = rng_for(w.seed)
    weights = draw_weights(rng, w.K, w.N)
    rows = 8 if name == "verify" else (M or w.M)
    x = draw_x(rng, rows, w.K, w.outlier_frac)
    m = M or w.M
    return Case(name, m, w.K, w.N, weights, np.ascontiguousarray(x[:m]))


def make_random(M: int, K: int, N: int, seed: int, outlier_frac: float = 0.0) -> Case:
    rng = rng_for(seed)
    weights = draw_weights(rng, K, N)
    x = draw_x(rng, M, K, outlier_frac)
    return Case(f"random_M{M}_K{K}_N{N}_s{seed}", M, K, N, weights, x)


def algorithmic_bytes(M: int, K: int, N: int) -> int:
    """Bytes one call must move: codes K*N/2, bf16 scale and minimum 4*N*K/128,
    bf16 x 2*M*K, fp32 y 4*M*N."""
    return K * N // 2 + 4 * N * (K // GROUP) + 2 * M * K + 4 * M * N

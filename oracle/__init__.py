"""fp64 CPU oracle for the int4-g128 asymmetric weight-streaming product.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and it
shares no code with that path: the only thing both sides take is the seeded
input generator in ``synth``, which holds none of the product's arithmetic.

The arithmetic lives in ``q4g128_oracle.c`` (plain C, fp64); this module only
marshals numpy arrays into it.  What it computes (Token Rush README, weight
format paragraph and bandwidth paragraph; bw24 article, exactness paragraph):

    q[n][k]  = nibble (k mod 8) of W[n][k // 8], low nibble first
    w[n][k]  = q[n][k] * scale[n][k // 128] + minimum[n][k // 128]   (exact, fp64)
    y[m][n]  = sum over k ascending of x[m][k] * w[n][k]               (fp64)
    a[m][n]  = sum over k of |x[m][k] * w[n][k]|                       (tolerance scale)
    w32      = w rounded once to fp32 (nearest, ties to even)

the quantizer that produces the format from bf16 weights (Token Rush README,
quantization section; the steps are in q4g128_oracle.c), and the epilogues
after the product (Token Rush README, steps table rows 3 and 8-9): SwiGLU on
a fused gate/up product and a residual add + RMSNorm.

bf16 tensors are passed as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libq4g128_oracle.so"
DEFAULT_LIB = os.path.join(_HERE, LIB_NAME)

STATUS = {0: "ok", 1: "invalid argument", 2: "fp64 dequant not exact", 3: "non-finite bf16 input"}


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes view of one compiled oracle library (the real one, or a copy
    built with a planted mistake for the pin tests)."""

    def __init__(self, path: str = DEFAULT_LIB):
        if not os.path.exists(path):
            raise OracleError(f"oracle library not built: {path} (run oracle.build.build_oracle())")
        self.path = path
        self.lib = ctypes.CDLL(path)
        L = self.lib
        vp, lg, ci = ctypes.c_void_p, ctypes.c_long, ctypes.c_int
        L.q4o_codes.argtypes = [vp, lg, lg, vp]
        L.q4o_dequant_f64.argtypes = [vp, vp, vp, lg, lg, vp]
        L.q4o_dequant_f32.argtypes = [vp, vp, vp, lg, lg, vp]
        L.q4o_gemm_cols.argtypes = [vp, lg, lg, vp, vp, vp, lg, vp, lg, vp, vp, ci]
        L.q4o_gemm.argtypes = [vp, lg, lg, vp, vp, vp, lg, vp, vp, ci]
        L.q4o_quantize.argtypes = [vp, lg, lg, ci, vp, vp, vp, vp, ci]
        L.q4o_swiglu.argtypes = [vp, lg, lg, vp]
        L.q4o_residual_rmsnorm.argtypes = [vp, vp, vp, ctypes.c_double, lg, lg, vp, vp]
        for f in ("q4o_codes", "q4o_dequant_f64", "q4o_dequant_f32", "q4o_gemm_cols",
                  "q4o_gemm", "q4o_quantize", "q4o_swiglu", "q4o_residual_rmsnorm", "q4o_abi_version", "q4o_plant", "q4o_max_threads"):
            getattr(L, f).restype = ci
        self.plant = L.q4o_plant()

    # -- argument checking (shapes only; values are the C side's business) --
    @staticmethod
    def _weights(W, scale, mn):
        W = np.ascontiguousarray(W, dtype=np.uint32)
        scale = np.ascontiguousarray(scale, dtype=np.uint16)
        mn = np.ascontiguousarray(mn, dtype=np.uint16)
        N, K8 = W.shape
        K = 8 * K8
        if scale.shape != (N, K // 128) or mn.shape != (N, K // 128):
            raise OracleError(f"scale/min shape {scale.shape}/{mn.shape} != {(N, K // 128)}")
        return W, scale, mn, K, N

    def _check(self, rc, what):
        if rc != 0:
            raise OracleError(f"{what}: {STATUS.get(rc, rc)}")

    def codes(self, W):
        W = np.ascontiguousarray(W, dtype=np.uint32)
        N, K8 = W.shape
        q = np.empty((N, 8 * K8), dtype=np.uint8)
        self._check(self.lib.q4o_codes(_ptr(W), 8 * K8, N, _ptr(q)), "codes")
        return q

    def dequant_f64(self, W, scale, mn):
        W, scale, mn, K, N = self._weights(W, scale, mn)
        w = np.empty((N, K), dtype=np.float64)
        self._check(self.lib.q4o_dequant_f64(_ptr(W), _ptr(scale), _ptr(mn), K, N, _ptr(w)), "dequant_f64")
        return w

    def dequant_f32(self, W, scale, mn):
        W, scale, mn, K, N = self._weights(W, scale, mn)
        w = np.empty((N, K), dtype=np.float32)
        self._check(self.lib.q4o_dequant_f32(_ptr(W), _ptr(scale), _ptr(mn), K, N, _ptr(w)), "dequant_f32")
        return w

    def gemm(self, x, W, scale, mn, cols=None, nthreads: int = 0):
        """Return (y, a), both fp64 [M][ncols] (ncols = N when cols is None)."""
        W, scale, mn, K, N = self._weights(W, scale, mn)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        if x.ndim != 2 or x.shape[1] != K:
            raise OracleError(f"x shape {x.shape} does not match K={K}")
        M = x.shape[0]
        if cols is None:
            y = np.empty((M, N), dtype=np.float64)
            a = np.empty((M, N), dtype=np.float64)
            rc = self.lib.q4o_gemm(_ptr(x), M, K, _ptr(W), _ptr(scale), _ptr(mn), N,
                                   _ptr(y), _ptr(a), int(nthreads))
        else:
            cols = np.ascontiguousarray(cols, dtype=np.int64)
            y = np.empty((M, cols.size), dtype=np.float64)
            a = np.empty((M, cols.size), dtype=np.float64)
            rc = self.lib.q4o_gemm_cols(_ptr(x), M, K, _ptr(W), _ptr(scale), _ptr(mn), N,
                                        _ptr(cols), cols.size, _ptr(y), _ptr(a), int(nthreads))
        self._check(rc, "gemm")
        return y, a

    def quantize(self, w, ncand: int = 9, nthreads: int = 0):
        """bf16 weights [N][K] (uint16 bit patterns) -> (W [N][K/8] uint32,
        scale [N][K/128] uint16, min [N][K/128] uint16, err [N][K/128] fp64):
        per-group range search: each end of the range clipped toward the middle by
        0, 1/20, .., (ncand-1)/20 of its half, ncand * ncand candidates (1 = round
        to nearest)."""
        w = np.ascontiguousarray(w, dtype=np.uint16)
        N, K = w.shape
        G = K // 128
        W = np.empty((N, K // 8), dtype=np.uint32)
        S = np.empty((N, G), dtype=np.uint16)
        Mn = np.empty((N, G), dtype=np.uint16)
        err = np.empty((N, G), dtype=np.float64)
        self._check(self.lib.q4o_quantize(_ptr(w), K, N, int(ncand), _ptr(W), _ptr(S), _ptr(Mn), _ptr(err),
                                          int(nthreads)), "quantize")
        return W, S, Mn, err

    def swiglu(self, y):
        """fp64 y [M][2I] (gate columns first, then up) -> act [M][I] = silu(g) * u."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        M, N = y.shape
        act = np.empty((M, N // 2), dtype=np.float64)
        self._check(self.lib.q4o_swiglu(_ptr(y), M, N, _ptr(act)), "swiglu")
        return act

    def residual_rmsnorm(self, y, r, gamma, eps: float):
        """fp64 y, r [M][N], gamma [N] bf16 bits -> (h = r + y, out = h / sqrt(mean(h^2) + eps) * gamma)."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        r = np.ascontiguousarray(r, dtype=np.float64)
        gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
        M, N = y.shape
        if r.shape != (M, N) or gamma.shape != (N,):
            raise OracleError(f"residual {r.shape} / gamma {gamma.shape} do not match y {y.shape}")
        h = np.empty((M, N), dtype=np.float64)
        out = np.empty((M, N), dtype=np.float64)
        self._check(self.lib.q4o_residual_rmsnorm(_ptr(y), _ptr(r), _ptr(gamma), float(eps), M, N, _ptr(h),
                                                  _ptr(out)), "residual_rmsnorm")
        return h, out

    def max_threads(self) -> int:
        return int(self.lib.q4o_max_threads())


_default = None


def load(path: str | None = None) -> Oracle:
    """The oracle built from q4g128_oracle.c (cached)."""
    global _default
    if path is not None:
        return Oracle(path)
    if _default is None:
        _default = Oracle(DEFAULT_LIB)
    return _default


def within_tolerance(y_test, y_ref, a_ref, rel: float = 1e-3, abs_: float = 1e-6):
    """Element-wise acceptance test |y - y_ref| <= rel * a + abs."""
    y_test = np.asarray(y_test, dtype=np.float64)
    return np.abs(y_test - y_ref) <= rel * a_ref + abs_

"""The product of a normalised input (q4g128_gemm_prenorm,
q4g128_gemm_swiglu_prenorm) and the residual-only form of
q4g128_gemm_rmsnorm, on MI355X through the C ABI.

  * x is made from fp32 rows h inside the product; the result equals, bit
    for bit, the product called on x_out = q4g128_gemm_rmsnorm's norm of the
    same h (taken with a zero product, so its h is h itself: the rows hold no
    negative zeros).  x_out is pinned to the oracle by the epilogue tests,
    the product by the parity tests, so this ties the fused path to both;
  * the one-launch form (x made while the balanced kernel stages it) and the
    form that writes x to the workspace first give the same bits; which one
    ran is read off the workspace (a sentinel the first leaves untouched);
  * rows bit-identical across M;
  * residual only (x_out NULL): h equals the h of the full call, in one
    launch and in two.
"""
import numpy as np
import pytest
import torch

import synth
import quantized_decode_q4g128_amd as q
from gpu_util import DEV, dev_weights, dev_x, host_f32

pytestmark = pytest.mark.gpu

SENTINEL = -7.0


def h_rows(M, K, seed):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((M, K)) * 1.5).astype(np.float32)
    h[h == 0] = 1.0                       # no zeros of either sign
    gamma = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(K))
    return h, gamma


def norm_ref(ht, gt, eps):
    """x_out of q4g128_gemm_rmsnorm for rows h: a zero product (all-zero
    codes, scales and minimums) plus the residual h."""
    M, K = ht.shape
    x0 = torch.zeros((M, 128), dtype=torch.int16, device=DEV)
    W0 = torch.zeros((K, 16), dtype=torch.int32, device=DEV)
    s0 = torch.zeros((K, 1), dtype=torch.int16, device=DEV)
    h, xo = q.q4g128_gemm_rmsnorm(x0, W0, s0, s0, ht, gt, eps, splits=1)
    assert np.array_equal(host_f32(h).view(np.uint32), host_f32(ht).view(np.uint32))
    return xo


def as_bits(t):
    torch.cuda.synchronize(DEV)
    return t.detach().cpu().view(torch.int16).numpy() if t.dtype != torch.float32 else \
        t.detach().cpu().numpy().view(np.uint32)


def run_prenorm(ht, gt, W, s, m, swiglu, eps=1e-6):
    M, K = ht.shape
    N = W.shape[0]
    nb = q.q4g128_prenorm_workspace_bytes(M, K, N, swiglu)
    ws = torch.full((nb // 4,), SENTINEL, dtype=torch.float32, device=DEV)
    f = q.q4g128_gemm_swiglu_prenorm if swiglu else q.q4g128_gemm_prenorm
    out = f(ht, gt, W, s, m, eps, workspace=ws)
    xwords = (M * K * 2 + 3) // 4
    one_launch = bool((ws[:xwords] == SENTINEL).all().item())
    return out, one_launch


# (M, K, N, swiglu, one launch expected: True / False / None = either)
CASES = [(1, 5120, 12288, False, True),      # q/k/v: register-ring kernel
         (1, 5120, 34816, True, True),       # gate/up + SwiGLU: LDS-fed kernel
         (6, 5120, 34816, True, True),       # verify rows: one launch up to 6
         (7, 5120, 34816, True, False),      # from 7 rows: a norm launch, then the product
         (8, 5120, 34816, True, False),
         (1, 5120, 32768, False, True),      # many tiles, plain
         (1, 6144, 5120, False, True),       # K parts
         (3, 6144, 5120, False, True),
         (4, 1024, 300, False, None), (3, 2048, 200, True, None), (1, 128, 2, True, None),
         (9, 5120, 12288, False, False)]     # more rows than the one-launch form takes


@pytest.mark.parametrize("M,K,N,swiglu,one", CASES)
def test_prenorm_equals_norm_then_product(M, K, N, swiglu, one):
    case = synth.make_random(1, K, N, 200 + M + N % 97)
    W, s, m = dev_weights(case.weights)
    h, gamma = h_rows(M, K, 300 + M)
    ht = torch.from_numpy(h).to(DEV)
    gt = torch.from_numpy(gamma.view(np.int16)).to(DEV)
    xo = norm_ref(ht, gt, 1e-6)
    ref = q.q4g128_gemm_swiglu(xo, W, s, m) if swiglu else q.q4g128_gemm(xo, W, s, m)
    got, one_launch = run_prenorm(ht, gt, W, s, m, swiglu)
    print(f"prenorm M={M} K={K} N={N} swiglu={swiglu}: {'one launch' if one_launch else 'two launches'}")
    if one is not None:
        assert one_launch == one
    assert np.array_equal(as_bits(got), as_bits(ref))


def test_prenorm_misaligned_h_takes_two_launches():
    case = synth.make_random(1, 5120, 12288, 210)
    W, s, m = dev_weights(case.weights)
    h, gamma = h_rows(2, 5120, 310)
    buf = torch.empty(2 * 5120 + 1, dtype=torch.float32, device=DEV)
    ht = buf[1:].view(2, 5120)
    ht.copy_(torch.from_numpy(h))
    gt = torch.from_numpy(gamma.view(np.int16)).to(DEV)
    got, one_launch = run_prenorm(ht, gt, W, s, m, False)
    assert not one_launch
    ref = q.q4g128_gemm(norm_ref(ht.contiguous().clone(), gt, 1e-6), W, s, m)
    assert np.array_equal(as_bits(got), as_bits(ref))


@pytest.mark.parametrize("K,N,swiglu", [(5120, 12288, False), (5120, 34816, True)])
def test_prenorm_rows_identical_across_M(K, N, swiglu):
    case = synth.make_random(1, K, N, 220)
    W, s, m = dev_weights(case.weights)
    h, gamma = h_rows(9, K, 320)
    gt = torch.from_numpy(gamma.view(np.int16)).to(DEV)
    full, _ = run_prenorm(torch.from_numpy(h).to(DEV), gt, W, s, m, swiglu)
    full = as_bits(full)
    for M in (1, 2, 5, 8):
        part, _ = run_prenorm(torch.from_numpy(h[:M].copy()).to(DEV), gt, W, s, m, swiglu)
        assert np.array_equal(as_bits(part), full[:M]), M


@pytest.mark.parametrize("M", [1, 2])
def test_residual_only_equals_full_h(M):
    """x_out NULL: h = residual + y alone, bit-equal to the h of the full
    call; one launch at M = 1 on 17408 -> 5120 (the workspace's partial
    area untouched), the partials path at M = 2."""
    case = synth.make_random(M, 17408, 5120, 230)
    W, s, m = dev_weights(case.weights)
    x = dev_x(case.x)
    rng = np.random.default_rng(330)
    r = (rng.standard_normal((M, 5120)) * 0.5).astype(np.float32)
    gamma = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(5120))
    gt = torch.from_numpy(gamma.view(np.int16)).to(DEV)
    P = q.q4g128_gemm_parts(17408, 5120)
    h_full, _ = q.q4g128_gemm_rmsnorm(x, W, s, m, torch.from_numpy(r).to(DEV), gt, 1e-6, splits=P)
    ws = q.q4g128_rmsnorm_workspace(M, 5120, P, DEV)
    ws[64:].fill_(SENTINEL)
    res = torch.from_numpy(r.copy()).to(DEV)
    h, none = q.q4g128_gemm_rmsnorm(x, W, s, m, res, None, splits=P, h=res, workspace=ws, norm=False)
    assert none is None and h.data_ptr() == res.data_ptr()
    assert np.array_equal(as_bits(h), as_bits(h_full))
    assert bool((ws[64:] == SENTINEL).all().item()) == (M == 1)
    assert not ws[:64].view(torch.int32).any().item()

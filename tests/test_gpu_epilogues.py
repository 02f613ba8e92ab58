"""The fused epilogues on MI355X, through the C ABI, against the oracle.

SwiGLU on a fused gate/up product (q4g128_gemm_swiglu):
  * within a tolerance derived from the product's bound: with tau = 1e-3 a +
    1e-6 per column, |silu'| <= 1.1, so |silu(g)u - silu(g*)u*| <= E =
    1.1 tau_g (|u*| + tau_u) + |silu(g*)| tau_u; fp32 arithmetic and the bf16
    rounding add at most 2^-8 (|act*| + E);
  * the one-launch path and the partials-then-activation path give the same
    bits (the second is taken when scale/min are not 16-byte aligned);
  * rows bit-identical across M; repeated calls identical.
Residual add + RMSNorm with split-K partials summed in the norm
(q4g128_gemm_rmsnorm):
  * h equals fp32(residual + y) bit for bit, y the split-K product with the
    same splits (q4g128_gemm_splitk);
  * x_out within a tolerance derived from h's bound (product bound plus one
    fp32 rounding), the fp32 sum of squares (at most ceil(N/8192) + 18
    sequential roundings: 8 in a block's chain, 4 in a group's tree,
    ceil(N/8192) in a lane's chain of group sums, 6 in the butterfly) and the
    correctly rounded sqrt and divide, plus 2^-8 relative for the fp32
    products and the bf16 rounding;
  * in place (h = residual) gives the same results; rows bit-identical
    across M; repeated calls identical;
  * the one-launch form (splits = the K parts, the last workgroup
    normalising) gives the bits of the two-launch form, and leaves the
    workspace's control block zero, call after call.
"""
import numpy as np
import pytest
import torch

import synth
import quantized_decode_q4g128_amd as q
from gpu_util import DEV, dev_weights, dev_x, host_f32

pytestmark = pytest.mark.gpu


def host_bf16(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize(DEV)
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def as_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def swiglu_tolerance(y_ref, a_ref):
    I = y_ref.shape[1] // 2
    tau = 1e-3 * a_ref + 1e-6
    g, u, tg, tu = y_ref[:, :I], y_ref[:, I:], tau[:, :I], tau[:, I:]
    silu = g / (1.0 + np.exp(-g))
    E = 1.1 * tg * (np.abs(u) + tu) + np.abs(silu) * tu
    return E + 2.0 ** -8 * (np.abs(silu * u) + E) + 1e-37


def assert_close(got, ref, tol, what):
    bad = ~(np.abs(got - ref) <= tol)
    if bad.any():
        m, n = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} outside tolerance; first ({m},{n}) got {got[m, n]!r} "
                             f"ref {ref[m, n]!r} tol {tol[m, n]!r}")
    return float(np.max(np.abs(got - ref) / tol))


def misaligned(t: torch.Tensor) -> torch.Tensor:
    """The same values at an address 2 bytes past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    view = buf[1:1 + t.numel()].view(t.shape)
    view.copy_(t)
    return view


SWIGLU_CASES = [("gateup", None, None, None, None), ("verify", None, None, None, None),
                (None, 3, 2048, 200, 81), (None, 1, 1024, 34, 82), (None, 2, 1024, 2, 83),
                (None, 8, 640, 100, 84), (None, 5, 8192, 778, 85), (None, 1, 17408, 2 * 1000, 86),
                (None, 9, 5120, 34816, 87), (None, 16, 2048, 2 * 1000, 88), (None, 13, 5120, 34816, 89)]


def swiglu_case(name, M, K, N, seed):
    if name == "verify":
        return synth.make_case("verify", 7)
    if name:
        return synth.make_case(name)
    return synth.make_random(M, K, N, seed)


@pytest.mark.parametrize("name,M,K,N,seed", SWIGLU_CASES)
def test_swiglu_within_tolerance(orc, name, M, K, N, seed):
    case = swiglu_case(name, M, K, N, seed)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    act_ref = orc.swiglu(y_ref)
    W, s, m = dev_weights(wt)
    act = as_f64(host_bf16(q.q4g128_gemm_swiglu(dev_x(case.x), W, s, m)))
    r = assert_close(act, act_ref, swiglu_tolerance(y_ref, a_ref), f"swiglu {case.name}")
    print(f"swiglu {case.name}: worst |err|/tol {r:.2e}")


@pytest.mark.parametrize("name,M,K,N,seed", SWIGLU_CASES[:4])
def test_swiglu_paths_agree(name, M, K, N, seed):
    case = swiglu_case(name, M, K, N, seed)
    x = dev_x(case.x)
    W, s, m = dev_weights(case.weights)
    fused = host_bf16(q.q4g128_gemm_swiglu(x, W, s, m))
    split = host_bf16(q.q4g128_gemm_swiglu(x, W, misaligned(s), misaligned(m)))
    assert np.array_equal(fused, split)
    again = host_bf16(q.q4g128_gemm_swiglu(x, W, s, m))
    assert np.array_equal(fused, again)


@pytest.mark.parametrize("K,N,seed", [(5120, 34816, 93), (4096, 33000, 94), (3072, 33000, 95)])
def test_swiglu_rows_identical_up_to_16_rows(K, N, seed):
    """Verify drafts of up to 15 tokens: gate/up + SwiGLU with x staged in
    chunks against x staged whole (5120: M <= 9, M = 8, 9 with ring slots
    for the tile waves only and one spare; 4096: that form at M = 10, 11;
    3072: at M = 14, 15)."""
    case = synth.make_random(16, K, N, seed)
    x16 = dev_x(case.x)
    W, s, m = dev_weights(case.weights)
    full = host_bf16(q.q4g128_gemm_swiglu(x16, W, s, m))
    for M in (1, 4, 8, 9, 10, 11, 12, 13, 14, 15):
        part = host_bf16(q.q4g128_gemm_swiglu(x16[:M].contiguous(), W, s, m))
        assert np.array_equal(part, full[:M]), M


@pytest.mark.parametrize("K,N,seed", [(5120, 34816, 3), (8192, 778, 91), (1024, 2, 92)])
def test_swiglu_rows_identical_across_M(K, N, seed):
    case = synth.make_random(8, K, N, seed)
    x8 = dev_x(case.x)
    W, s, m = dev_weights(case.weights)
    full = host_bf16(q.q4g128_gemm_swiglu(x8, W, s, m))
    for M in range(1, 8):
        part = host_bf16(q.q4g128_gemm_swiglu(x8[:M].contiguous(), W, s, m))
        assert np.array_equal(part, full[:M]), M


def rms_inputs(case, seed):
    rng = np.random.default_rng(seed)
    r = (rng.standard_normal((case.M, case.N)) * 0.5).astype(np.float32)
    gamma = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(case.N))
    return r, gamma


def rms_tolerance(y_ref, a_ref, r, gamma_bits, eps, out_ref):
    N = y_ref.shape[1]
    tau = 1e-3 * a_ref + 1e-6
    h = r.astype(np.float64) + y_ref
    th = tau + 2.0 ** -24 * (np.abs(h) + tau)
    ss = np.sum(h * h, axis=1, keepdims=True)
    L = -(-N // 8192) + 18
    dss = np.sum(2 * np.abs(h) * th + th * th, axis=1, keepdims=True) + (L + 3) * 2.0 ** -24 * ss
    inv = 1.0 / np.sqrt(ss / N + eps)
    d = 1.01 * 0.5 * dss / (ss + N * eps) + 4 * 2.0 ** -24
    gm = np.abs(as_f64(gamma_bits))[None, :]
    E = gm * (th * inv * (1 + d) + np.abs(h) * inv * d)
    return E + 2.0 ** -8 * (np.abs(out_ref) + E) + 1e-37


RMS_CASES = [("down", None, None, None, None, None), ("down", None, None, None, None, 1),
             (None, 3, 6144, 5120, 95, None), (None, 2, 1024, 1000, 96, None), (None, 1, 2048, 20000, 97, None),
             (None, 8, 1024, 300, 98, None), (None, 1, 128, 1, 99, None), (None, 16, 17408, 5120, 100, None),
             (None, 9, 6144, 5120, 101, None)]


def rms_case(name, M, K, N, seed):
    return synth.make_case(name) if name else synth.make_random(M, K, N, seed)


@pytest.mark.parametrize("name,M,K,N,seed,splits", RMS_CASES)
def test_rmsnorm_against_oracle(orc, name, M, K, N, seed, splits):
    case = rms_case(name, M, K, N, seed)
    wt = case.weights
    r, gamma = rms_inputs(case, 7)
    eps = 1e-6
    x = dev_x(case.x)
    W, s, m = dev_weights(wt)
    rt = torch.from_numpy(r).to(DEV)
    gt = torch.from_numpy(gamma.view(np.int16)).to(DEV)
    S = splits or q.q4g128_splitk_default_splits(case.K, case.N)
    h, xo = q.q4g128_gemm_rmsnorm(x, W, s, m, rt, gt, eps, splits=S)
    h, xo = host_f32(h), as_f64(host_bf16(xo))
    y_split = host_f32(q.q4g128_gemm_splitk(x, W, s, m, splits=S))
    assert np.array_equal(h.view(np.uint32), (r + y_split).view(np.uint32)), "h != fp32(r + y)"
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    _, out_ref = orc.residual_rmsnorm(y_ref, r.astype(np.float64), gamma, eps)
    worst = assert_close(xo, out_ref, rms_tolerance(y_ref, a_ref, r, gamma, eps, out_ref), f"rmsnorm {case.name}")
    print(f"rmsnorm {case.name} S={S}: worst |err|/tol {worst:.2e}")


def test_rmsnorm_in_place_and_repeatable():
    case = synth.make_case("down")
    r, gamma = rms_inputs(case, 8)
    x = dev_x(case.x)
    W, s, m = dev_weights(case.weights)
    gt = torch.from_numpy(gamma.view(np.int16)).to(DEV)
    h1, x1 = q.q4g128_gemm_rmsnorm(x, W, s, m, torch.from_numpy(r).to(DEV), gt)
    h1, x1 = host_f32(h1), host_bf16(x1)
    res = torch.from_numpy(r.copy()).to(DEV)
    h2, x2 = q.q4g128_gemm_rmsnorm(x, W, s, m, res, gt, h=res)
    assert h2.data_ptr() == res.data_ptr()
    assert np.array_equal(host_f32(res).view(np.uint32), h1.view(np.uint32))
    assert np.array_equal(host_bf16(x2), x1)


@pytest.mark.parametrize("K,N,seed", [(17408, 5120, 2), (1024, 300, 101)])
def test_rmsnorm_rows_identical_across_M(K, N, seed):
    case = synth.make_random(8, K, N, seed)
    rng = np.random.default_rng(102)
    r = rng.standard_normal((8, N)).astype(np.float32)
    gamma = synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(N))
    x8 = dev_x(case.x)
    W, s, m = dev_weights(case.weights)
    gt = torch.from_numpy(gamma.view(np.int16)).to(DEV)
    hf, xf = q.q4g128_gemm_rmsnorm(x8, W, s, m, torch.from_numpy(r).to(DEV), gt)
    hf, xf = host_f32(hf), host_bf16(xf)
    for M in (1, 2, 5, 7):
        h, xo = q.q4g128_gemm_rmsnorm(x8[:M].contiguous(), W, s, m, torch.from_numpy(r[:M].copy()).to(DEV), gt)
        assert np.array_equal(host_f32(h).view(np.uint32), hf[:M].view(np.uint32)), M
        assert np.array_equal(host_bf16(xo), xf[:M]), M


def rms_two_launch(x, W, s, m, r, g, S):
    """The two-launch form on the same operands: scale/min copied to
    addresses that are not 16-byte aligned, which the one-launch kernel does
    not take (same values, so the same split-K partials)."""
    return q.q4g128_gemm_rmsnorm(x, W, misaligned(s), misaligned(m), r, g, 1e-6, splits=S)


@pytest.mark.parametrize("name,M,K,N,seed", [("down", None, None, None, None), (None, 1, 6144, 5120, 103),
                                             (None, 4, 6144, 5120, 104), (None, 8, 6144, 5120, 105)])
def test_rmsnorm_one_launch_equals_two_launch(name, M, K, N, seed):
    case = rms_case(name, M, K, N, seed)
    P = q.q4g128_gemm_parts(case.K, case.N)
    assert P > 1, "a shape the one-launch form serves"
    r, gamma = rms_inputs(case, 9)
    x = dev_x(case.x)
    W, s, m = dev_weights(case.weights)
    rt = torch.from_numpy(r).to(DEV)
    gt = torch.from_numpy(gamma.view(np.int16)).to(DEV)
    ws = q.q4g128_rmsnorm_workspace(case.M, case.N, P, DEV)
    ws[64:].fill_(-7.0)                         # the partials area: untouched by the one-launch form
    h1, x1 = q.q4g128_gemm_rmsnorm(x, W, s, m, rt, gt, 1e-6, splits=P, workspace=ws)
    h1, x1 = host_f32(h1), host_bf16(x1)
    one_launch = bool((ws[64:] == -7.0).all().item())
    if case.M == 1:
        assert one_launch, "M = 1 on a K-part shape runs as one launch"
    print(f"rmsnorm {case.name} M={case.M} P={P}: {'one launch' if one_launch else 'two launches'}")
    h2, x2 = rms_two_launch(x, W, s, m, rt, gt, P)
    assert np.array_equal(h1.view(np.uint32), host_f32(h2).view(np.uint32))
    assert np.array_equal(x1, host_bf16(x2))
    # the counter in the control block is back at zero, and a reused
    # workspace gives the same bits (also in place, h = residual)
    assert not ws[:64].view(torch.int32).any().item()
    for _ in range(3):
        res = torch.from_numpy(r.copy()).to(DEV)
        h3, x3 = q.q4g128_gemm_rmsnorm(x, W, s, m, res, gt, 1e-6, splits=P, h=res, workspace=ws)
        assert np.array_equal(host_f32(h3).view(np.uint32), h1.view(np.uint32))
        assert np.array_equal(host_bf16(x3), x1)
    assert not ws[:64].view(torch.int32).any().item()


def test_rmsnorm_one_launch_shared_workspace_across_shapes():
    """One workspace serving the one-launch form and the two-launch form in
    turn (down projection at M = 1, then at M = 2, which its LDS does not
    hold): the two-launch form leaves the control block alone."""
    case = synth.make_random(2, 17408, 5120, 106)
    P = q.q4g128_gemm_parts(case.K, case.N)
    r, gamma = rms_inputs(case, 10)
    x = dev_x(case.x)
    W, s, m = dev_weights(case.weights)
    rt = torch.from_numpy(r).to(DEV)
    gt = torch.from_numpy(gamma.view(np.int16)).to(DEV)
    ws = q.q4g128_rmsnorm_workspace(2, case.N, P, DEV)
    ref = []
    for M in (1, 2, 1, 2):
        ws[64:].fill_(-7.0)
        h, xo = q.q4g128_gemm_rmsnorm(x[:M].contiguous(), W, s, m, rt[:M].contiguous(), gt, 1e-6, splits=P,
                                      workspace=ws)
        ref.append((host_f32(h).view(np.uint32), host_bf16(xo)))
        assert not ws[:64].view(torch.int32).any().item(), M
        assert bool((ws[64:] == -7.0).all().item()) == (M == 1), M      # M = 2: partials written
    assert np.array_equal(ref[0][0], ref[2][0]) and np.array_equal(ref[0][1], ref[2][1])
    assert np.array_equal(ref[1][0], ref[3][0]) and np.array_equal(ref[1][1], ref[3][1])
    assert np.array_equal(ref[1][0][:1], ref[0][0]) and np.array_equal(ref[1][1][:1], ref[0][1])

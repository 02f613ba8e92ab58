"""Every launch form the dispatch can choose, reached and checked: for a grid
of (K, N) shapes, every M from 1 to 16 must run (status OK) and give rows
bit-identical to the 16-row call's, for the plain product, the split-K call
with its default split count and the fused SwiGLU product.

The grid reaches, by K and the tiles each workgroup holds at 256 compute
units: the LDS-fed burst form with every wave's ring slots (all M at 2048 ->
33000), with the deep ring (M <= 4), with the tile waves' slots and one
spare (M = 14, 15 at 3072; 10, 11 at 4096; 8, 9 at 5120), x staged first
(M = 16 at 3072), x in chunks (M >= 12 at 4096, >= 10 at 5120, >= 9 at
6144 and 8192), the register-ring kernel (7 tiles, and K = 1024), K parts
held in one launch or in row blocks (5120 -> 20480 / 12288, 6144 -> 5120,
8192 -> 777, 17408 -> 5120), the split-K call's partial sums and reduce,
and the per-tile kernel (N = 100).

Inputs are drawn on the device from a seeded generator (random code words;
bf16 x ~ N(0, 1), scale |N(0, 1)| * 0.01 + 1e-4, minimum -8 * scale + N(0,
1e-3)); the test compares the library with itself, so no oracle is needed.
"""
import pytest
import torch

import quantized_decode_q4g128_amd as q
from gpu_util import DEV

pytestmark = pytest.mark.gpu

SHAPES = [(1024, 12288), (2048, 33000), (3072, 33000), (4096, 33000), (5120, 34816), (6144, 33001),
          (8192, 33000), (5120, 28672), (5120, 20480), (5120, 12288), (6144, 5120), (17408, 5120),
          (8192, 777), (1024, 100)]


def device_case(K, N, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    W = torch.randint(-2 ** 31, 2 ** 31 - 1, (N, K // 8), dtype=torch.int32, device=DEV, generator=g)
    s = torch.randn((N, K // 128), device=DEV, generator=g).abs() * 0.01 + 1e-4
    m = -8.0 * s.to(torch.bfloat16).float() + 1e-3 * torch.randn((N, K // 128), device=DEV, generator=g)
    x = torch.randn((16, K), device=DEV, generator=g)
    return x.to(torch.bfloat16), W, s.to(torch.bfloat16).contiguous(), m.to(torch.bfloat16).contiguous()


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                       b.contiguous().view(torch.int32 if b.dtype == torch.float32 else torch.int16))


@pytest.mark.parametrize("K,N", SHAPES)
def test_every_row_count_runs_and_keeps_rows(K, N):
    x, W, s, m = device_case(K, N, 1000 + K // 128 + N % 997)
    calls = [("gemm", lambda xx: q.q4g128_gemm(xx, W, s, m)),
             ("splitk", lambda xx: q.q4g128_gemm_splitk(xx, W, s, m))]
    if N % 2 == 0:
        calls.append(("swiglu", lambda xx: q.q4g128_gemm_swiglu(xx, W, s, m)))
    for name, f in calls:
        full = f(x)
        torch.cuda.synchronize(DEV)
        for M in range(1, 16):
            part = f(x[:M].contiguous())
            assert same_bits(part, full[:M]), f"{name} K={K} N={N} M={M}"
    torch.cuda.synchronize(DEV)


@pytest.mark.parametrize("K,N", SHAPES)
def test_fused_norm_entries_keep_rows(K, N):
    """The same for the entries with a norm: the product of RMSNorm(h) made
    inside the launch (plain and SwiGLU; M <= 8 in one launch, the
    normalised x through the workspace beyond) and h = r + y with and
    without x_out = RMSNorm(h) (K-part shapes in one launch where the rows
    fit, partial sums and one norm launch otherwise): each row depends on its
    own inputs only, so every output must equal the 16-row call's rows."""
    _, W, s, m = device_case(K, N, 2000 + K // 128 + N % 997)
    g = torch.Generator(device=DEV)
    g.manual_seed(3000 + K // 128 + N % 997)
    hin = torch.randn((16, K), device=DEV, generator=g) * 3.0
    gk = (1.0 + 0.1 * torch.randn((K,), device=DEV, generator=g)).to(torch.bfloat16)
    xr = torch.randn((16, K), device=DEV, generator=g).to(torch.bfloat16)
    res = torch.randn((16, N), device=DEV, generator=g)
    gn = (1.0 + 0.1 * torch.randn((N,), device=DEV, generator=g)).to(torch.bfloat16)
    calls = [("prenorm", lambda M: (q.q4g128_gemm_prenorm(hin[:M].contiguous(), gk, W, s, m),)),
             ("rmsnorm", lambda M: q.q4g128_gemm_rmsnorm(xr[:M].contiguous(), W, s, m, res[:M].contiguous(), gn)),
             ("residual", lambda M: q.q4g128_gemm_rmsnorm(xr[:M].contiguous(), W, s, m, res[:M].contiguous(), gn,
                                                         norm=False)[:1])]
    if N % 2 == 0:
        calls.append(("swiglu_prenorm", lambda M: (q.q4g128_gemm_swiglu_prenorm(hin[:M].contiguous(), gk, W, s, m),)))
    for name, f in calls:
        full = f(16)
        torch.cuda.synchronize(DEV)
        for M in range(1, 16):
            part = f(M)
            for j, (a, b) in enumerate(zip(part, full)):
                assert same_bits(a, b[:M]), f"{name} output {j} K={K} N={N} M={M}"
    torch.cuda.synchronize(DEV)

"""Host threads: the library's entry points called from several threads at
once, each on a stream of its own, give the bits of the same calls made one
after another.  The calls take different shapes and kernels (the LDS-fed
burst form, K parts in one launch, split-K partial sums and their reduce,
the fused SwiGLU, the residual add with RMSNorm), so the per-device caches
the library fills on first use (compute-unit count, each kernel's LDS room)
are read and filled from several threads.  ctypes releases the interpreter
lock for the duration of each call."""
import threading

import pytest
import torch

import quantized_decode_q4g128_amd as q
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def device_case(M, K, N, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    W = torch.randint(-2 ** 31, 2 ** 31 - 1, (N, K // 8), dtype=torch.int32, device=DEV, generator=g)
    s = torch.randn((N, K // 128), device=DEV, generator=g).abs() * 0.01 + 1e-4
    m = -8.0 * s.to(torch.bfloat16).float() + 1e-3 * torch.randn((N, K // 128), device=DEV, generator=g)
    x = torch.randn((M, K), device=DEV, generator=g).to(torch.bfloat16)
    r = torch.randn((M, N), device=DEV, generator=g)
    gamma = (1.0 + 0.1 * torch.randn((N,), device=DEV, generator=g)).to(torch.bfloat16)
    return x, W, s.to(torch.bfloat16).contiguous(), m.to(torch.bfloat16).contiguous(), r, gamma


def jobs():
    out = []
    for i, (M, K, N, kind) in enumerate([(1, 5120, 34816, "gemm"), (3, 17408, 5120, "splitk"),
                                         (7, 6144, 5120, "splitk"), (9, 5120, 12288, "gemm"),
                                         (2, 5120, 34816, "swiglu"), (1, 17408, 5120, "rmsnorm"),
                                         (8, 3072, 33000, "gemm"), (5, 1024, 1000, "splitk")]):
        x, W, s, m, r, gamma = device_case(M, K, N, 500 + i)

        def call(stream, x=x, W=W, s=s, m=m, r=r, gamma=gamma, kind=kind):
            if kind == "gemm":
                return (q.q4g128_gemm(x, W, s, m, stream=stream),)
            if kind == "splitk":
                return (q.q4g128_gemm_splitk(x, W, s, m, stream=stream),)
            if kind == "swiglu":
                return (q.q4g128_gemm_swiglu(x, W, s, m, stream=stream),)
            return q.q4g128_gemm_rmsnorm(x, W, s, m, r, gamma, stream=stream)
        out.append(call)
    return out


def as_bits(t):
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def test_host_threads_give_sequential_bits():
    calls = jobs()
    ref = [[as_bits(t).clone() for t in c(torch.cuda.current_stream(DEV))] for c in calls]
    torch.cuda.synchronize(DEV)
    results = [None] * len(calls)
    errors = []

    def worker(i):
        try:
            st = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(st):
                for _ in range(25):
                    outs = calls[i](st)
                st.synchronize()
            results[i] = [as_bits(t).clone() for t in outs]
            st.synchronize()
        except Exception as e:                      # reported below, with the job index
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(calls))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize(DEV)
    for i, (a, b) in enumerate(zip(results, ref)):
        assert a is not None, i
        for j, (u, v) in enumerate(zip(a, b)):
            assert torch.equal(u, v), f"job {i} output {j}"

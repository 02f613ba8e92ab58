"""The C ABI under HIP graph capture: launches recorded once (no memsets,
no allocations inside the calls) replay to the eager results, bit for bit,
with eager work and synchronisation between the replays."""
import numpy as np
import pytest
import torch

import synth
import quantized_decode_q4g128_amd as q
from gpu_util import DEV, bits, dev_weights, dev_x, host_f32

pytestmark = pytest.mark.gpu


def test_graph_replay_equals_eager():
    cases = [synth.make_random(1, 5120, 4096, 51),        # balanced kernel
             synth.make_random(3, 17408, 640, 52),        # per-tile kernel with split-K + reduce
             synth.make_random(2, 6144, 1000, 53)]        # balanced kernel with K parts
    ops = []
    for c in cases:
        x = dev_x(c.x)
        W, s, m = dev_weights(c.weights)
        y = torch.empty((c.M, c.N), dtype=torch.float32, device=DEV)
        splits = q.q4g128_splitk_default_splits(c.K, c.N)
        ws = torch.empty(max(4, q.q4g128_splitk_workspace_bytes(c.M, c.N, splits)) // 4, dtype=torch.float32,
                         device=DEV)
        ops.append((x, W, s, m, y, splits, ws))

    def run_all(stream=None):
        for x, W, s, m, y, splits, ws in ops:
            q.q4g128_gemm_splitk(x, W, s, m, splits=splits, workspace=ws, y=y, stream=stream)

    run_all()
    torch.cuda.synchronize()
    eager = [host_f32(op[4]) for op in ops]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all(torch.cuda.current_stream())
    for rep in range(3):
        for op in ops:
            op[4].fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, op in enumerate(ops):
            assert np.array_equal(bits(host_f32(op[4])), bits(eager[k])), (rep, k)
        del junk


def test_graph_replay_of_fused_epilogues_equals_eager():
    """SwiGLU (one-launch and partials forms) and the residual-add + RMSNorm
    (in place on the residual, which every replay restores first)."""
    gu = synth.make_random(1, 5120, 4096, 54)              # balanced kernel, SwiGLU in the same launch
    gp = synth.make_random(3, 640, 200, 55)                # K not a multiple of 1024: partials + sum_swiglu
    dn = synth.make_random(2, 17408, 1024, 56)             # split-K by the default count, norm over N = 1024
    rng = np.random.default_rng(57)
    r0 = torch.from_numpy(rng.standard_normal((dn.M, dn.N)).astype(np.float32)).to(DEV)
    gamma = torch.from_numpy(synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(dn.N)).view(np.int16)).to(DEV)
    ops = []
    for c in (gu, gp):
        x = dev_x(c.x)
        W, s, m = dev_weights(c.weights)
        act = torch.empty((c.M, c.N // 2), dtype=torch.bfloat16, device=DEV)
        ws = torch.empty(max(4, q.q4g128_swiglu_workspace_bytes(c.M, c.K, c.N)) // 4, dtype=torch.float32,
                         device=DEV)
        ops.append(("swiglu", x, W, s, m, act, ws))
    xd = dev_x(dn.x)
    Wd, sd, md = dev_weights(dn.weights)
    S = q.q4g128_splitk_default_splits(dn.K, dn.N)
    h = r0.clone()
    xo = torch.empty((dn.M, dn.N), dtype=torch.bfloat16, device=DEV)
    wsd = q.q4g128_rmsnorm_workspace(dn.M, dn.N, S, DEV)

    def run_all(stream=None):
        for _, x, W, s, m, act, ws in ops:
            q.q4g128_gemm_swiglu(x, W, s, m, act=act, workspace=ws, stream=stream)
        q.q4g128_gemm_rmsnorm(xd, Wd, sd, md, h, gamma, 1e-6, splits=S, h=h, x_out=xo, workspace=wsd, stream=stream)

    def outs():
        torch.cuda.synchronize()
        return [o[5].view(torch.int16).cpu().numpy() for o in ops] + [host_f32(h).view(np.uint32),
                                                                       xo.view(torch.int16).cpu().numpy()]

    h.copy_(r0)
    run_all()
    eager = outs()
    g = torch.cuda.CUDAGraph()
    h.copy_(r0)
    with torch.cuda.graph(g):
        run_all(torch.cuda.current_stream())
    for rep in range(3):
        for o in ops:
            o[5].fill_(float("nan"))
        xo.fill_(float("nan"))
        h.copy_(r0)                                          # the residual the graph updates in place
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        got = outs()
        for k, (a, b) in enumerate(zip(got, eager)):
            assert np.array_equal(a, b), (rep, k)
        del junk

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


def test_graph_replay_of_norm_forms_equals_eager():
    """The one-launch residual + RMSNorm (its workgroups count themselves in
    the workspace's control block; the last one normalises and clears it),
    the residual add alone, and products that normalise their input (q/k/v
    and gate/up + SwiGLU from fp32 rows), chained as in a decoder layer."""
    dn = synth.make_random(1, 17408, 5120, 58)             # one launch: K parts of the LDS-fed kernel
    qk = synth.make_random(1, 5120, 12288, 59)             # q/k/v shape: register-ring kernel
    gu = synth.make_random(1, 5120, 34816, 60)             # gate/up + SwiGLU: LDS-fed kernel
    rng = np.random.default_rng(61)
    r1 = torch.from_numpy(rng.standard_normal((1, 5120)).astype(np.float32)).to(DEV)
    r2 = torch.from_numpy(rng.standard_normal((1, 5120)).astype(np.float32)).to(DEV)
    gamma = torch.from_numpy(synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(5120)).view(np.int16)).to(DEV)
    xd = dev_x(dn.x)
    Wd, sd, md = dev_weights(dn.weights)
    Wq, sq, mq = dev_weights(qk.weights)
    Wg, sg, mg = dev_weights(gu.weights)
    P = q.q4g128_gemm_parts(17408, 5120)
    h1, h2 = r1.clone(), r2.clone()
    xo = torch.empty((1, 5120), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((1, 12288), dtype=torch.float32, device=DEV)
    act = torch.empty((1, 17408), dtype=torch.bfloat16, device=DEV)
    wn1 = q.q4g128_rmsnorm_workspace(1, 5120, P, DEV)
    wn2 = q.q4g128_rmsnorm_workspace(1, 5120, P, DEV)
    wp = torch.empty(max(q.q4g128_prenorm_workspace_bytes(1, 5120, 12288),
                         q.q4g128_prenorm_workspace_bytes(1, 5120, 34816, True)) // 4, dtype=torch.float32, device=DEV)

    def run_all(stream=None):
        q.q4g128_gemm_rmsnorm(xd, Wd, sd, md, h1, gamma, 1e-6, splits=P, h=h1, x_out=xo, workspace=wn1, stream=stream)
        q.q4g128_gemm_rmsnorm(xd, Wd, sd, md, h2, None, splits=P, h=h2, workspace=wn2, stream=stream, norm=False)
        q.q4g128_gemm_prenorm(h2, gamma, Wq, sq, mq, 1e-6, y=y, workspace=wp, stream=stream)
        q.q4g128_gemm_swiglu_prenorm(h1, gamma, Wg, sg, mg, 1e-6, act=act, workspace=wp, stream=stream)

    def outs():
        torch.cuda.synchronize()
        return [host_f32(h1).view(np.uint32), host_f32(h2).view(np.uint32), xo.view(torch.int16).cpu().numpy(),
                host_f32(y).view(np.uint32), act.view(torch.int16).cpu().numpy()]

    h1.copy_(r1)
    h2.copy_(r2)
    run_all()
    eager = outs()
    g = torch.cuda.CUDAGraph()
    h1.copy_(r1)
    h2.copy_(r2)
    with torch.cuda.graph(g):
        run_all(torch.cuda.current_stream())
    for rep in range(3):
        for t in (xo, y, act):
            t.fill_(float("nan"))
        h1.copy_(r1)
        h2.copy_(r2)
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        got = outs()
        for k, (a, b) in enumerate(zip(got, eager)):
            assert np.array_equal(a, b), (rep, k)
        assert not wn1[:64].view(torch.int32).any().item()
        del junk

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

"""Parity of the work-balanced (stream-K) entry point with the fp64 oracle.

Tiles split between waves are summed in a fixed part order by the last wave
to finish them, through a per-tile counter in a zero-filled workspace that
every call leaves zero-filled.  Covered: every workload within tolerance,
rows bit-identical across M = 1..8 (one and two K slices), repeated calls on
one workspace (counters reset), heavily split tiles, ragged N, exact
power-of-two scaling, and argument errors.
"""
import numpy as np
import pytest
import torch

import synth
import quantized_decode_q4g128_amd as q
from gpu_util import DEV, assert_within_tolerance, bits, dev_weights, dev_x, host_f32

pytestmark = pytest.mark.gpu


def run_sk(case_x, wt, ws=None):
    return host_f32(q.q4g128_gemm_streamk(dev_x(case_x), *dev_weights(wt), workspace=ws))


@pytest.mark.parametrize("name", ["tiny", "gateup", "down", "verify"])
def test_workloads_within_tolerance(orc, name):
    case = synth.make_case(name)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    r = assert_within_tolerance(run_sk(case.x, wt), y_ref, a_ref, f"{name} streamk")
    print(f"{name}: worst |err|/tol {r:.2e}")


@pytest.mark.parametrize("K,N,seed", [(K, N, sd) for K, N, sd in synth.stream_shapes()])
def test_stream_shapes_within_tolerance(orc, K, N, seed):
    case = synth.make_random(1, K, N, seed)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    assert_within_tolerance(run_sk(case.x, wt), y_ref, a_ref, f"stream K={K} N={N}")


@pytest.mark.parametrize("K,N,seed", [(5120, 34816, 3), (17408, 5120, 2)])
def test_rows_bit_identical_across_M(K, N, seed):
    case = synth.make_random(8, K, N, seed, outlier_frac=0.01)
    W, s, m = dev_weights(case.weights)
    x8 = dev_x(case.x)
    ws = q.q4g128_streamk_workspace(K, N, DEV)
    y8 = host_f32(q.q4g128_gemm_streamk(x8, W, s, m, workspace=ws))
    for M in range(1, 8):
        yM = host_f32(q.q4g128_gemm_streamk(x8[:M].contiguous(), W, s, m, workspace=ws))
        assert np.array_equal(bits(yM), bits(y8[:M])), M
    for r in (0, 3, 7):
        y1 = host_f32(q.q4g128_gemm_streamk(x8[r:r + 1].contiguous(), W, s, m, workspace=ws))
        assert np.array_equal(bits(y1[0]), bits(y8[r])), r


def test_workspace_reused_across_calls_and_inputs(orc):
    # One workspace, several different products in a row: if a counter were
    # left non-zero, a later call would finish its tiles early or never.
    K, N = 5120, 2000
    ws = q.q4g128_streamk_workspace(K, N, DEV)
    first = None
    for seed in (40, 41, 40, 42):
        case = synth.make_random(3, K, N, seed)
        wt = case.weights
        y = run_sk(case.x, wt, ws)
        y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
        assert_within_tolerance(y, y_ref, a_ref, f"seed {seed}")
        if seed == 40:
            if first is None:
                first = y
            else:
                assert np.array_equal(bits(first), bits(y))      # deterministic
    # Counters follow 2 MiB of part slots; every call leaves them at zero.
    tiles = (N + 15) // 16
    part_words = 2 * 2048 * 128
    cnt = ws.view(torch.int32)[part_words:part_words + tiles].cpu().numpy()
    assert (cnt == 0).all()


@pytest.mark.parametrize("M,K,N", [(1, 17408, 16), (8, 17408, 16), (3, 5120, 48), (2, 1024, 1),
                                   (8, 1024, 17), (5, 2048, 100), (4, 6144, 1000), (7, 9216, 333)])
def test_split_tiles_and_ragged_shapes(orc, M, K, N):
    case = synth.make_random(M, K, N, 200 + M + N, outlier_frac=0.01)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    assert_within_tolerance(run_sk(case.x, wt), y_ref, a_ref, f"M={M} K={K} N={N}")


def test_power_of_two_scaling_is_exact():
    case = synth.make_random(3, 5120, 777, 9)
    W, s, m = dev_weights(case.weights)
    x2 = case.x.copy()
    nz = (x2 & 0x7F80) != 0
    x2[nz] += 0x0080
    ws = q.q4g128_streamk_workspace(5120, 777, DEV)
    y = host_f32(q.q4g128_gemm_streamk(dev_x(case.x), W, s, m, workspace=ws))
    y2 = host_f32(q.q4g128_gemm_streamk(dev_x(x2), W, s, m, workspace=ws))
    assert np.array_equal(bits(y2), bits(2 * y))


def test_unsupported_and_invalid_arguments():
    wide = synth.make_random(9, 1024, 16, 5)         # stream-K keeps M <= 8
    with pytest.raises(q.Q4G128Error) as e:
        q.q4g128_gemm_streamk(dev_x(wide.x), *dev_weights(wide.weights))
    assert e.value.status == q.Q4G128_EINVAL
    case = synth.make_random(1, 640, 8, 5)           # K not a multiple of 1024
    with pytest.raises(ValueError):
        q.q4g128_gemm_streamk(dev_x(case.x), *dev_weights(case.weights))
    case = synth.make_random(1, 1024, 8, 5)
    small = torch.zeros(16, dtype=torch.int32, device=DEV)
    with pytest.raises(q.Q4G128Error) as e:
        q.q4g128_gemm_streamk(dev_x(case.x), *dev_weights(case.weights), workspace=small)
    assert e.value.status == q.Q4G128_EWORKSPACE

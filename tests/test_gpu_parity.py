"""Parity of the HIP path (through the C ABI) with the fp64 oracle on MI355X.

* dequant export: bit-exact against the oracle's once-rounded weights;
* one-hot activations select single weights (ties the product's unpack to
  the oracle's);
* every workload within |y - y_ref| <= 1e-3 * sum|x*w| + 1e-6;
* rows of an M-row call bit-identical to one-row calls, M = 1..16;
* split-K deterministic run to run and across streams;
* y(2x) = 2 y(x) exactly;
* ragged and extreme shapes.
"""
import numpy as np
import pytest
import torch

import synth
import quantized_decode_q4g128_amd as q
from gpu_util import DEV, assert_within_tolerance, bits, dev_weights, dev_x, host_f32

pytestmark = pytest.mark.gpu


def test_device_is_gfx950():
    assert torch.cuda.is_available()
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name


@pytest.mark.parametrize("K,N,seed", [(1024, 1024, 0), (256, 17, 1), (128, 1, 2), (5120, 64, 3),
                                      (17408, 5, 4)])
def test_dequant_bit_exact(orc, K, N, seed):
    case = synth.make_random(1, K, N, seed)
    wt = case.weights
    w = host_f32(q.q4g128_dequant(*dev_weights(wt)))
    w32 = orc.dequant_f32(wt.W, wt.scale, wt.mn)
    assert np.array_equal(bits(w), bits(w32))


def test_one_hot_selects_weights(orc):
    K, N = 1024, 100
    case = synth.make_random(1, K, N, 7)
    wt = case.weights
    w32 = orc.dequant_f32(wt.W, wt.scale, wt.mn)
    ks = [0, 1, 4, 7, 8, 130, 515, 1023]           # every nibble slot, several groups
    x = np.zeros((8, K), dtype=np.uint16)
    for m, k in enumerate(ks):
        x[m, k] = 0x3F80
    y = host_f32(q.q4g128_gemm(dev_x(x), *dev_weights(wt)))
    s = synth.bf16_bits_to_f32(wt.scale).astype(np.float64)
    mn = synth.bf16_bits_to_f32(wt.mn).astype(np.float64)
    madj = mn - 128.0 * s                           # exact in fp64
    madj_exact = madj.astype(np.float32).astype(np.float64) == madj
    for m, k in enumerate(ks):
        g = k // 128
        exact_cols = madj_exact[:, g]
        assert exact_cols.mean() > 0.9
        assert np.array_equal(bits(y[m, exact_cols]), bits(w32[exact_cols, k])), (m, k)
        # where mn - 128*s rounds in fp32, the result is still within one rounding
        ok = np.abs(y[m, ~exact_cols] - w32[~exact_cols, k]) <= 2 ** -22 * np.abs(w32[~exact_cols, k]) + 1e-30
        assert ok.all(), (m, k)


WORKLOADS = ["tiny", "gateup", "down", "verify"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_within_tolerance(orc, name):
    case = synth.make_case(name)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    x = dev_x(case.x)
    W, s, m = dev_weights(wt)
    y = host_f32(q.q4g128_gemm(x, W, s, m))
    r1 = assert_within_tolerance(y, y_ref, a_ref, f"{name} gemm")
    ys = host_f32(q.q4g128_gemm_splitk(x, W, s, m))
    r2 = assert_within_tolerance(ys, y_ref, a_ref, f"{name} gemm_splitk")
    print(f"{name}: worst |err|/tol gemm {r1:.2e} splitk {r2:.2e}")


@pytest.mark.parametrize("K,N,seed", [(K, N, sd) for K, N, sd in synth.stream_shapes()])
def test_stream_shapes_within_tolerance(orc, K, N, seed):
    case = synth.make_random(1, K, N, seed)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    x = dev_x(case.x)
    W, s, m = dev_weights(wt)
    y = host_f32(q.q4g128_gemm_splitk(x, W, s, m))
    assert_within_tolerance(y, y_ref, a_ref, f"stream K={K} N={N}")


def test_rows_bit_identical_to_single_row_verify_shape():
    case = synth.make_case("verify", 8)
    W, s, m = dev_weights(case.weights)
    x8 = dev_x(case.x)
    y8 = host_f32(q.q4g128_gemm(x8, W, s, m))
    for M in range(1, 9):
        yM = host_f32(q.q4g128_gemm(x8[:M].contiguous(), W, s, m))
        assert np.array_equal(bits(yM), bits(y8[:M])), M
    for r in range(8):
        y1 = host_f32(q.q4g128_gemm(x8[r:r + 1].contiguous(), W, s, m))
        assert np.array_equal(bits(y1[0]), bits(y8[r])), r


def test_rows_bit_identical_to_single_row_split_k():
    case = synth.make_random(8, 17408, 5120, 2, outlier_frac=0.01)
    W, s, m = dev_weights(case.weights)
    x8 = dev_x(case.x)
    y8 = host_f32(q.q4g128_gemm_splitk(x8, W, s, m))
    for M in (1, 2, 3, 5, 7):
        yM = host_f32(q.q4g128_gemm_splitk(x8[:M].contiguous(), W, s, m))
        assert np.array_equal(bits(yM), bits(y8[:M])), M
    for r in range(8):
        y1 = host_f32(q.q4g128_gemm_splitk(x8[r:r + 1].contiguous(), W, s, m))
        assert np.array_equal(bits(y1[0]), bits(y8[r])), r


def test_rows_bit_identical_when_x_is_staged_in_chunks():
    # K = 17408 without a split: one LDS stage at M = 1, 2; several chunks for
    # M >= 3.  The chunking must not change any bit.
    case = synth.make_random(8, 17408, 1000, 12, outlier_frac=0.01)
    W, s, m = dev_weights(case.weights)
    x8 = dev_x(case.x)
    y8 = host_f32(q.q4g128_gemm(x8, W, s, m))
    for M in range(1, 8):
        yM = host_f32(q.q4g128_gemm(x8[:M].contiguous(), W, s, m))
        assert np.array_equal(bits(yM), bits(y8[:M])), M


def test_split_k_deterministic_across_runs_and_streams():
    case = synth.make_case("down")
    W, s, m = dev_weights(case.weights)
    x = dev_x(case.x)
    ya = host_f32(q.q4g128_gemm_splitk(x, W, s, m))
    yb = host_f32(q.q4g128_gemm_splitk(x, W, s, m))
    side = torch.cuda.Stream(DEV)
    with torch.cuda.stream(side):
        yc_t = q.q4g128_gemm_splitk(x, W, s, m, stream=side)
    side.synchronize()
    yc = host_f32(yc_t)
    assert np.array_equal(bits(ya), bits(yb)) and np.array_equal(bits(ya), bits(yc))
    y1 = host_f32(q.q4g128_gemm_splitk(x, W, s, m, splits=1))
    yg = host_f32(q.q4g128_gemm(x, W, s, m))
    assert np.array_equal(bits(y1), bits(yg))


# More splits than 1024-k blocks: up to one split per 128-group, cut at group
# boundaries (K = 17408: 17 blocks, 136 groups).  Each split count stays
# within the tolerance, repeats its bits on another run and on another
# stream, and keeps rows bit-identical to one-row calls.
@pytest.mark.parametrize("splits", [17, 34, 136])
def test_split_k_up_to_one_split_per_group(orc, splits):
    case = synth.make_random(3, 17408, 5120, 2, outlier_frac=0.01)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    W, s, m = dev_weights(wt)
    x = dev_x(case.x)
    ya = host_f32(q.q4g128_gemm_splitk(x, W, s, m, splits=splits))
    r = assert_within_tolerance(ya, y_ref, a_ref, f"splits={splits}")
    yb = host_f32(q.q4g128_gemm_splitk(x, W, s, m, splits=splits))
    side = torch.cuda.Stream(DEV)
    with torch.cuda.stream(side):
        yc_t = q.q4g128_gemm_splitk(x, W, s, m, splits=splits, stream=side)
    side.synchronize()
    yc = host_f32(yc_t)
    assert np.array_equal(bits(ya), bits(yb)) and np.array_equal(bits(ya), bits(yc))
    for row in range(3):
        y1 = host_f32(q.q4g128_gemm_splitk(x[row:row + 1].contiguous(), W, s, m, splits=splits))
        assert np.array_equal(bits(y1[0]), bits(ya[row])), row
    print(f"splits={splits}: worst |err|/tol {r:.2e}")


# Group-granular splits of short K, ragged split widths (K = 640: 5 groups
# in one block) and K not a multiple of 1024.
@pytest.mark.parametrize("M,K,N,splits", [(2, 640, 100, 5), (2, 640, 100, 3), (1, 1152, 33, 9), (4, 3200, 70, 7)])
def test_split_k_group_granular_edges(orc, M, K, N, splits):
    case = synth.make_random(M, K, N, 140 + K // 128 + splits, outlier_frac=0.01)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    y = host_f32(q.q4g128_gemm_splitk(dev_x(case.x), *dev_weights(wt), splits=splits))
    assert_within_tolerance(y, y_ref, a_ref, f"M={M} K={K} N={N} splits={splits}")


@pytest.mark.parametrize("splits", [None, 1])
def test_power_of_two_scaling_is_exact(splits):
    case = synth.make_random(3, 5120, 777, 9)
    W, s, m = dev_weights(case.weights)
    x2 = case.x.copy()
    nz = (x2 & 0x7F80) != 0
    x2[nz] += 0x0080                                # doubles every normal bf16
    assert ((x2 & 0x7FFF)[~nz] == 0).all()          # no subnormals in the draw
    f = q.q4g128_gemm if splits == 1 else q.q4g128_gemm_splitk
    y = host_f32(f(dev_x(case.x), W, s, m))
    y2 = host_f32(f(dev_x(x2), W, s, m))
    assert np.array_equal(bits(y2), bits(2 * y))


EDGE = [(1, 128, 1), (3, 128, 17), (8, 256, 100), (2, 1024, 1000), (8, 17408, 48), (5, 384, 65),
        (1, 2048, 16), (4, 640, 63)]


@pytest.mark.parametrize("M,K,N", EDGE)
def test_edge_shapes(orc, M, K, N):
    case = synth.make_random(M, K, N, 100 + M + K + N, outlier_frac=0.01)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    x = dev_x(case.x)
    W, s, m = dev_weights(wt)
    G = K // 128
    assert_within_tolerance(host_f32(q.q4g128_gemm(x, W, s, m)), y_ref, a_ref, "gemm")
    nb = (G + 7) // 8
    for sp in sorted({1, 2, 3, nb} & set(range(1, nb + 1))):
        y = host_f32(q.q4g128_gemm_splitk(x, W, s, m, splits=sp))
        assert_within_tolerance(y, y_ref, a_ref, f"splitk splits={sp}")


def test_output_fully_overwritten(orc):
    case = synth.make_random(2, 4096, 40, 77)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    y = torch.full((2, 40), float("nan"), dtype=torch.float32, device=DEV)   # K=4096: 4 blocks
    q.q4g128_gemm(dev_x(case.x), *dev_weights(wt), y=y)
    assert_within_tolerance(host_f32(y), y_ref, a_ref, "prefilled y")
    y.fill_(float("nan"))
    q.q4g128_gemm_splitk(dev_x(case.x), *dev_weights(wt), splits=4, y=y)
    assert_within_tolerance(host_f32(y), y_ref, a_ref, "prefilled y split")


def test_invalid_arguments_are_rejected_before_launch():
    case = synth.make_random(1, 256, 8, 5)
    W, s, m = dev_weights(case.weights)
    x = dev_x(case.x)
    with pytest.raises(q.Q4G128Error) as e:
        q.q4g128_gemm_splitk(x, W, s, m, splits=3)      # K=256 holds two 128-groups
    assert e.value.status == q.Q4G128_EINVAL
    with pytest.raises(q.Q4G128Error) as e:
        q.q4g128_gemm(dev_x(np.zeros((17, 256), np.uint16)), W, s, m)
    assert e.value.status == q.Q4G128_EINVAL
    big = synth.make_random(1, 2048, 8, 6)
    ws = torch.empty(4, dtype=torch.float32, device=DEV)
    with pytest.raises(q.Q4G128Error) as e:
        q.q4g128_gemm_splitk(dev_x(big.x), *dev_weights(big.weights), splits=2, workspace=ws)
    assert e.value.status == q.Q4G128_EWORKSPACE
    with pytest.raises(ValueError):
        q.q4g128_gemm(x[:, :128].contiguous(), W, s, m)


# Rows of every M must be the same bits whichever kernel serves M: at
# K = 7168, N = 32768 the balanced kernel takes M <= 6 and the per-tile
# kernel M = 7, 8 (x no longer fits the balanced staging); at K = 6144 and
# 8192 with small N the choice covers every M alike (K parts / per-tile).
@pytest.mark.parametrize("K,N", [(7168, 32768), (6144, 1000), (8192, 777)])
def test_rows_bit_identical_across_kernel_choice(K, N):
    case = synth.make_random(8, K, N, 31 + K // 1024)
    W, s, m = dev_weights(case.weights)
    x8 = dev_x(case.x)
    y8 = host_f32(q.q4g128_gemm(x8, W, s, m))
    for M in range(1, 8):
        yM = host_f32(q.q4g128_gemm(x8[:M].contiguous(), W, s, m))
        assert np.array_equal(bits(yM), bits(y8[:M])), M


# Verify wider than 8 rows (a draft of up to 15 tokens plus the next one):
# rows of every M up to 16 equal the 16-row call's.  At K = 5120, N = 34816
# the LDS-fed kernel takes M <= 9 with x staged whole (M = 8, 9 with ring
# slots for the tile waves only and one spare) and M >= 10 with x in chunks
# (loaded by the waves without a tile); at K =
# 8192, N = 777 the balanced kernel cuts K into 8 parts and holds 6 rows per
# launch; 17408 -> 5120 (6 parts) runs with its default splits (one LDS-fed
# launch for M = 1, 6 K splits and their sum beyond); 6144 -> 5120 (6 parts,
# 8 rows per launch) without splits; 5120 -> 12288 (3 parts) and 5120 ->
# 20480 (2 parts) in row blocks of 9.  1024 -> 12288 (3 tiles per CU, no
# block to cut: the register-ring kernel loads one group per load, all 16
# rows in one launch) and 5120 -> 28672 (7 tiles per CU: two groups per load,
# M <= 9; the chunked form for M >= 10) cover both load patterns of the
# register-ring kernel, and M = 3,
# 4, 5, 12, 13 cross the 1-, 2-, 3- and 4-row accumulation of the balanced
# kernels.  4096 -> 33000 (9 tiles per CU) takes the burst form with every
# wave's slots for M <= 9, the one with the tile waves' slots and a shared
# spare for M = 10, 11 (3 accumulated rows), and x in chunks from M = 12.
# 3072 -> 33000 takes that form at M = 14, 15 (4 accumulated rows).  6144 ->
# 33001 (9 tiles, the last workgroup's ragged) stages x in chunks from M = 9
# (its x no longer fits the staging registers whole).
@pytest.mark.parametrize("K,N,split", [(5120, 34816, False), (8192, 777, False), (17408, 5120, True),
                                       (6144, 5120, False), (5120, 12288, False), (5120, 20480, False),
                                       (1024, 12288, False), (5120, 28672, False), (4096, 33000, False),
                                       (6144, 33001, False), (3072, 33000, False)])
def test_rows_bit_identical_up_to_16_rows(K, N, split):
    case = synth.make_random(16, K, N, 60 + K // 1024 + N % 1000, outlier_frac=0.01)
    W, s, m = dev_weights(case.weights)
    x16 = dev_x(case.x)
    f = q.q4g128_gemm_splitk if split else q.q4g128_gemm
    y16 = host_f32(f(x16, W, s, m))
    for M in (1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13, 14, 15):
        yM = host_f32(f(x16[:M].contiguous(), W, s, m))
        assert np.array_equal(bits(yM), bits(y16[:M])), M


@pytest.mark.parametrize("M,K,N", [(8, 5120, 34816), (9, 5120, 34816), (16, 5120, 34816), (9, 17408, 5120),
                                   (16, 2048, 1001),
                                   (13, 1024, 17), (16, 640, 100), (11, 4096, 33000), (12, 6144, 33001),
                                   (14, 3072, 33000)])
def test_wide_verify_within_tolerance(orc, M, K, N):
    case = synth.make_random(M, K, N, 70 + M, outlier_frac=0.01)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    x = dev_x(case.x)
    W, s, m = dev_weights(wt)
    r1 = assert_within_tolerance(host_f32(q.q4g128_gemm(x, W, s, m)), y_ref, a_ref, f"M={M} K={K} N={N}")
    r2 = assert_within_tolerance(host_f32(q.q4g128_gemm_splitk(x, W, s, m)), y_ref, a_ref, f"split M={M}")
    print(f"M={M} K={K} N={N}: worst |err|/tol {r1:.2e} / split-K {r2:.2e}")


# Column sharing of the balanced kernel: N not a multiple of 8, fewer than 8
# columns per CU, one tile per wave with an 8-column tail, and more tiles per
# workgroup than waves (several tiles per wave).
@pytest.mark.parametrize("M,N", [(1, 1001), (3, 200), (1, 7), (2, 34816), (1, 131072), (5, 50000)])
def test_balanced_column_sharing(orc, M, N):
    K = 1024 if N > 40000 else 2048
    case = synth.make_random(M, K, N, 40 + M + N % 97)
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    y = host_f32(q.q4g128_gemm(dev_x(case.x), *dev_weights(wt)))
    assert_within_tolerance(y, y_ref, a_ref, f"balanced M={M} N={N}")


def _misaligned(t):
    buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    view = buf[1:1 + t.numel()].view(t.shape)
    view.copy_(t)
    return view


# K-part shapes: one balanced launch whose parts are the blocks of P K splits
# gives the bits of the per-tile kernel with P splits and the split-order
# reduce (forced here by scales/minimums off a 16-byte boundary), for the
# rows one launch holds and beyond.
@pytest.mark.parametrize("K,N", [(17408, 5120), (6144, 5120), (8192, 777)])
def test_k_parts_equal_split_k(K, N):
    case = synth.make_random(8, K, N, 120 + K // 1024, outlier_frac=0.01)
    W, s, m = dev_weights(case.weights)
    S = q.q4g128_gemm_parts(K, N)
    assert S >= 2
    for M in (1, 2, 3, 8):
        x = dev_x(case.x[:M])
        fast = host_f32(q.q4g128_gemm_splitk(x, W, s, m, splits=S))
        tile = host_f32(q.q4g128_gemm_splitk(x, W, _misaligned(s), _misaligned(m), splits=S))
        plain = host_f32(q.q4g128_gemm(x, W, s, m))
        assert np.array_equal(bits(fast), bits(tile)), (M, "parts vs splits")
        assert np.array_equal(bits(fast), bits(plain)), (M, "splits vs no split")


# Deep ring of the LDS-fed kernel's whole-K burst form (rows 1-4 only): with
# 8 tiles per CU (4 waves without a tile) at K = 2048 the youngest tile
# wave's 8-pair ring covers its unit exactly; 9 tiles at K = 3072 leave a
# partial second pass (12 pairs); K = 1024 (4 pairs) is too short for it.
# Rows 1-4 must equal the 5-row call's rows, which never takes the deep ring,
# and the 4-row call must be within tolerance; the SwiGLU form alike.
@pytest.mark.parametrize("K,N", [(2048, 32768), (3072, 34816), (1024, 34816)])
def test_deep_ring_rows_equal_plain_ring(orc, K, N):
    case = synth.make_random(5, K, N, 90 + K // 1024, outlier_frac=0.01)
    wt = case.weights
    W, s, m = dev_weights(wt)
    x5 = dev_x(case.x)
    y5 = host_f32(q.q4g128_gemm(x5, W, s, m))
    a5 = q.q4g128_gemm_swiglu(x5, W, s, m).view(torch.int16).cpu().numpy()
    for M in (1, 2, 3, 4):
        xM = x5[:M].contiguous()
        assert np.array_equal(bits(host_f32(q.q4g128_gemm(xM, W, s, m))), bits(y5[:M])), M
        assert np.array_equal(q.q4g128_gemm_swiglu(xM, W, s, m).view(torch.int16).cpu().numpy(), a5[:M]), M
    y_ref, a_ref = orc.gemm(case.x[:4], wt.W, wt.scale, wt.mn)
    assert_within_tolerance(y5[:4], y_ref, a_ref, f"deep ring K={K} N={N}")

"""More of the C ABI on MI355X: a row slice of a larger table (the draft's
partial-vocabulary output projection), calls in flight on two streams at
once, and weights and activations far from the usual magnitudes."""
import numpy as np
import pytest
import torch

import synth
import quantized_decode_q4g128_amd as q
from gpu_util import DEV, assert_within_tolerance, bits, dev_weights, dev_x, host_f32

pytestmark = pytest.mark.gpu


def test_row_slice_of_a_larger_table(orc):
    """The draft reads a 131072-row slice of a 248320-row output projection
    (Token Rush README, steps table row 20): the product on the slice's rows
    equals the same columns of the whole table's product bit for bit (the
    per-column sums do not depend on N here), and sampled columns match the
    oracle."""
    K, N_full, r0, n = 5120, 248320, 65536, 131072
    case = synth.make_random(1, K, N_full, 111)
    W, s, m = dev_weights(case.weights)
    x = dev_x(case.x)
    y_full = host_f32(q.q4g128_gemm(x, W, s, m))
    Ws, ss, ms = (t[r0:r0 + n] for t in (W, s, m))          # contiguous row slices (views)
    assert Ws.is_contiguous() and Ws.data_ptr() % 16 == 0
    y_slice = host_f32(q.q4g128_gemm(x, Ws, ss, ms))
    assert np.array_equal(bits(y_slice), bits(y_full[:, r0:r0 + n]))
    cols = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(112).choice(n, 254, replace=False)]))
    wt = case.weights
    y_ref, a_ref = orc.gemm(case.x, wt.W[r0:r0 + n], wt.scale[r0:r0 + n], wt.mn[r0:r0 + n], cols=cols)
    assert_within_tolerance(y_slice[:, cols], y_ref, a_ref, "lm_head slice")


def test_calls_in_flight_on_two_streams():
    """Split-K products on two streams at once, each with its own workspace,
    give the bits of the same calls made one after the other."""
    a = synth.make_case("down")
    b = synth.make_random(3, 5120, 12288, 113)
    ops = []
    for c in (a, b):
        x = dev_x(c.x)
        W, s, m = dev_weights(c.weights)
        S = q.q4g128_splitk_default_splits(c.K, c.N)
        ws = torch.empty(max(4, q.q4g128_splitk_workspace_bytes(c.M, c.N, S)) // 4, dtype=torch.float32, device=DEV)
        ops.append((x, W, s, m, S, ws, torch.empty((c.M, c.N), dtype=torch.float32, device=DEV)))
    seq = []
    for x, W, s, m, S, ws, y in ops:
        q.q4g128_gemm_splitk(x, W, s, m, splits=S, workspace=ws, y=y)
        seq.append(host_f32(y).copy())
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    torch.cuda.synchronize()
    for rep in range(5):
        for (x, W, s, m, S, ws, y), st in zip(ops, (s1, s2)):
            with torch.cuda.stream(st):
                y.fill_(float("nan"))
                q.q4g128_gemm_splitk(x, W, s, m, splits=S, workspace=ws, y=y, stream=st)
        torch.cuda.synchronize()
        for k, op in enumerate(ops):
            assert np.array_equal(bits(host_f32(op[6])), bits(seq[k])), (rep, k)


@pytest.mark.parametrize("sscale,xscale", [(1e-4, 1e3), (1e3, 1e-4), (2.0 ** -100, 2.0 ** 60)])
def test_far_magnitudes(orc, sscale, xscale):
    """Scales and minimums 1e-4..1e3 times the usual, activations scaled the
    other way (and by powers of two far from 1): within tolerance, and for
    the power-of-two case bit-exactly the usual result rescaled."""
    K, N = 2048, 500
    rng = synth.rng_for(114)
    wt = synth.draw_weights(rng, K, N)
    xb = synth.draw_x(rng, 2, K)
    sf = synth.bf16_bits_to_f32(wt.scale).astype(np.float64) * sscale
    mf = synth.bf16_bits_to_f32(wt.mn).astype(np.float64) * sscale
    xf = synth.bf16_bits_to_f32(xb).astype(np.float64) * xscale
    w2 = synth.Weights(wt.W, synth.to_bf16_bits(sf), synth.to_bf16_bits(mf))
    x2 = synth.to_bf16_bits(xf)
    y = host_f32(q.q4g128_gemm(dev_x(x2), *dev_weights(w2)))
    y_ref, a_ref = orc.gemm(x2, w2.W, w2.scale, w2.mn)
    assert_within_tolerance(y, y_ref, a_ref, f"s x {sscale:g}, x x {xscale:g}")
    if sscale == 2.0 ** -100:                     # exact power-of-two rescaling of every operand
        y0 = host_f32(q.q4g128_gemm(dev_x(xb), *dev_weights(wt)))
        assert np.array_equal(bits(y), bits((y0.astype(np.float64) * sscale * xscale).astype(np.float32)))

"""The GPU quantizer (q4g128_quantize, through the C ABI) against the
oracle's quantizer on MI355X: codes, scale, minimum and each group's squared
error bit for bit, for round-to-nearest and for the range search; special
groups; non-finite groups; a sampled check at a full projection shape; and
the quantized weights feeding the product."""
import numpy as np
import pytest
import torch

import synth
import quantized_decode_q4g128_amd as q
from gpu_util import DEV, assert_within_tolerance, bits, dev_x, host_f32

pytestmark = pytest.mark.gpu


def dev_w(w_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(w_bits).view(np.int16)).to(DEV)


def host(outs):
    torch.cuda.synchronize(DEV)
    W, s, m, e = (t.cpu().numpy() for t in outs)
    return W.view(np.uint32), s.view(np.uint16), m.view(np.uint16), e


def assert_same(gpu, ref, what):
    W, s, m, e = gpu
    Wr, sr, mr, er = ref
    for name, a, b in (("codes", W, Wr), ("scale", s, sr), ("min", m, mr)):
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{what}: {name} differs at {len(bad)} places, first {tuple(bad[0])}")
    assert np.array_equal(e.view(np.uint64), er.view(np.uint64)), f"{what}: error sums differ"


@pytest.mark.parametrize("ncand", [1, 2, 3, 9, 16])
@pytest.mark.parametrize("N,K,seed", [(40, 1024, 11), (7, 384, 12), (1, 128, 13)])
def test_quantize_bit_exact(orc, ncand, N, K, seed):
    w = synth.draw_dense_weights(synth.rng_for(seed), N, K, outlier_frac=3e-3)
    gpu = host(q.q4g128_quantize(dev_w(w), ncand))
    assert_same(gpu, orc.quantize(w, ncand), f"N={N} K={K} ncand={ncand}")


def special_groups():
    """One row of 128-weight groups that exercise the corner cases."""
    rng = np.random.default_rng(21)
    rows = []
    rows.append(np.full(128, 0.375))                                  # constant
    rows.append(np.zeros(128))                                        # all zero
    z = np.zeros(128); z[::2] = -0.0; rows.append(z)                   # signed zeros
    rows.append((rng.integers(0, 16, 128) - 8) * 2.0 ** -6)           # already on a grid
    rows.append(rng.standard_normal(128) * 1e-30)                     # tiny magnitudes
    rows.append(rng.standard_normal(128) * 1e30)                      # huge magnitudes
    o = rng.standard_normal(128) * 0.01; o[5] = 3.0; rows.append(o)   # one far outlier
    o = rng.standard_normal(128) * 0.01; o[9] = -3.0; o[77] = 2.0; rows.append(o)
    t = np.linspace(-1, 1, 128); rows.append(t)                       # evenly spread
    rows.append(np.where(np.arange(128) % 2 == 0, 1.0, -1.0))         # two values
    h = (np.arange(128) % 31) * 2.0 ** -5                              # half steps of 1/16 over [0, 15/16]:
    h[0], h[1] = 0.0, 15.0 / 16.0                                      # exact ties at every odd multiple
    rows.append(h)
    rows.append(-3.0 + h * 4.0)                                        # the same ties, shifted and scaled
    return synth.to_bf16_bits(np.concatenate(rows)[None, :])


@pytest.mark.parametrize("ncand", [1, 9, 16])
def test_quantize_special_groups(orc, ncand):
    w = special_groups()
    gpu = host(q.q4g128_quantize(dev_w(w), ncand))
    assert_same(gpu, orc.quantize(w, ncand), f"special groups, ncand={ncand}")


def test_quantize_nonfinite_group(orc):
    """A group holding NaN or infinity: zero codes, scale and min, err NaN;
    every other group as the oracle quantizes it."""
    w = synth.draw_dense_weights(synth.rng_for(31), 4, 512)
    w[1, 130] = 0x7FC0          # NaN in group 1 of row 1
    w[3, 511] = 0xFF80          # -inf in group 3 of row 3
    W, s, m, e = host(q.q4g128_quantize(dev_w(w), 9))
    for (n, g) in ((1, 1), (3, 3)):
        assert np.isnan(e[n, g])
        assert np.all(W[n, 16 * g:16 * g + 16] == 0) and s[n, g] == 0 and m[n, g] == 0
    for n in (0, 2):
        ref = orc.quantize(w[n:n + 1], 9)
        assert_same((W[n:n + 1], s[n:n + 1], m[n:n + 1], e[n:n + 1]), ref, f"row {n}")
    for n, g in ((1, 0), (1, 2), (1, 3), (3, 0), (3, 1), (3, 2)):
        ref = orc.quantize(np.ascontiguousarray(w[n:n + 1, 128 * g:128 * g + 128]), 9)
        got = (W[n:n + 1, 16 * g:16 * g + 16], s[n:n + 1, g:g + 1], m[n:n + 1, g:g + 1], e[n:n + 1, g:g + 1])
        assert_same(got, ref, f"row {n} group {g}")


def test_quantize_full_shape_sampled(orc):
    """The down-projection shape (K=17408, N=5120) quantized whole on the GPU;
    the oracle checks every group of 48 sampled columns, first and last
    included."""
    N, K = 5120, 17408
    w = synth.draw_dense_weights(synth.rng_for(41), N, K)
    gpu = host(q.q4g128_quantize(dev_w(w), 9))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(42).choice(N, 46, replace=False)]))
    ref = orc.quantize(np.ascontiguousarray(w[rows]), 9)
    assert_same(tuple(a[rows] for a in gpu), ref, "down shape, sampled columns")


def test_quantized_weights_feed_the_product(orc):
    """Quantize on the GPU, then run the product on the result: the dequant
    export equals the oracle's dequant of the oracle's quantization, and the
    product is within tolerance of the oracle's product."""
    N, K = 300, 2048
    rng = synth.rng_for(51)
    w = synth.draw_dense_weights(rng, N, K)
    x = synth.draw_x(rng, 3, K)
    Wd, sd, md, _ = q.q4g128_quantize(dev_w(w), 9)
    Wr, sr, mr, _ = orc.quantize(w, 9)
    wd = host_f32(q.q4g128_dequant(Wd, sd, md))
    assert np.array_equal(bits(wd), bits(orc.dequant_f32(Wr, sr, mr)))
    y = host_f32(q.q4g128_gemm(dev_x(x), Wd, sd, md))
    y_ref, a_ref = orc.gemm(x, Wr, sr, mr)
    assert_within_tolerance(y, y_ref, a_ref, "quantize -> gemm")

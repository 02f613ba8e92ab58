"""q4g128_gemm_splitk_noalloc (partials in the library's own device scratch)
against q4g128_gemm_splitk (partials in a caller workspace): the same kernels,
so the same bits, on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

import synth
import quantized_decode_q4g128_amd as q
from gpu_util import DEV, bits, dev_weights, dev_x, host_f32

pytestmark = pytest.mark.gpu


def _pair(M, K, N, seed, splits):
    case = synth.make_random(M, K, N, seed, outlier_frac=0.01)
    W, s, m = dev_weights(case.weights)
    x = dev_x(case.x)
    ref = host_f32(q.q4g128_gemm_splitk(x, W, s, m, splits=splits))
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.q4g128_gemm_splitk_noalloc(x, W, s, m, y, splits=splits)
    return ref, host_f32(y)


@pytest.mark.parametrize("first,second", [
    ((4, 17408, 5120, 6), (1, 17408, 5120, 6)),       # down projection: default split count, fewer rows
    ((3, 6144, 4000, 40), (2, 2048, 300, 11)),        # group-granular splits, then a smaller shape
])
def test_noalloc_equals_workspace_path(first, second):
    for i, (M, K, N, splits) in enumerate((first, second)):
        ref, got = _pair(M, K, N, 300 + i, splits)
        assert np.array_equal(bits(got), bits(ref)), (M, K, N, splits)


def test_noalloc_rejects_oversize_scratch():
    case = synth.make_random(16, 17408, 5120, 9)
    W, s, m = dev_weights(case.weights)
    y = torch.empty((16, 5120), dtype=torch.float32, device=DEV)
    with pytest.raises(q.Q4G128Error) as e:
        q.q4g128_gemm_splitk_noalloc(dev_x(case.x), W, s, m, y, splits=136)
    assert e.value.status == q.Q4G128_EWORKSPACE

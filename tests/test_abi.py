"""The C-ABI library without a GPU: it loads, exports every function
include/q4g128.h declares, and rejects bad arguments before launching
anything (every call below returns before its first HIP call)."""
import ctypes
import os
import re

import pytest

import quantized_decode_q4g128_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4g128.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4g128_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(q.LIB_PATH):
        pytest.fail("libq4g128.so is not built (run __graft_entry__.build())")
    return q.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert {"q4g128_gemm", "q4g128_gemm_splitk", "q4g128_dequant"} <= set(names)
    for name in names:
        assert hasattr(L, name), f"{name} declared in q4g128.h but not exported"


def test_version_and_status_strings(L):
    assert q.q4g128_abi_version() == 1
    assert q.q4g128_status_string(0) == "ok"
    assert q.q4g128_status_string(1) == "invalid argument"
    assert q.q4g128_status_string(2) == "workspace too small"
    assert q.q4g128_status_string(3) == "HIP error"
    assert q.q4g128_status_string(99) == "unknown status"


def test_gemm_parts_arguments(L):
    assert q.q4g128_gemm_parts(100, 10) == 0 and q.q4g128_gemm_parts(1024, 0) == 0
    assert q.q4g128_gemm_parts(640, 100) == 1                 # K not a multiple of 1024: never cut


def test_workspace_bytes(L):
    assert q.q4g128_splitk_workspace_bytes(1, 5120, 7) == 7 * 5120 * 4
    assert q.q4g128_splitk_workspace_bytes(8, 34816, 2) == 2 * 8 * 34816 * 4
    for bad in ((0, 10, 2), (17, 10, 2), (1, 0, 2), (1, 10, 0)):
        assert q.q4g128_splitk_workspace_bytes(*bad) == 0


def test_default_splits_depend_on_shape_only(L):
    # Wide N needs no split; short N is split to fill the machine; never more
    # splits than 128-groups.
    assert q.q4g128_splitk_default_splits(5120, 34816) == 1
    assert q.q4g128_splitk_default_splits(5120, 131072) == 1
    s_down = q.q4g128_splitk_default_splits(17408, 5120)
    assert 2 <= s_down <= 17                  # at most one split per 1024 k
    assert q.q4g128_splitk_default_splits(1024, 1024) == 1
    assert q.q4g128_splitk_default_splits(128, 1) == 1
    assert q.q4g128_splitk_default_splits(100, 10) == 0
    assert q.q4g128_splitk_default_splits(1024, 0) == 0


FAKE = 0x10000   # 64 KiB-aligned non-null address; never dereferenced


def call_gemm(L, x=FAKE, M=1, K=256, W=FAKE, s=FAKE, m=FAKE, N=16, y=FAKE):
    return L.q4g128_gemm(x, M, K, W, s, m, N, y, None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(W=None), dict(s=None), dict(m=None), dict(y=None),
    dict(M=0), dict(M=17), dict(K=0), dict(K=100), dict(K=-128), dict(N=0),
    dict(x=FAKE + 8), dict(W=FAKE + 4), dict(s=FAKE + 1), dict(y=FAKE + 2),
])
def test_gemm_rejects(L, kw):
    assert call_gemm(L, **kw) == q.Q4G128_EINVAL


def test_splitk_rejects(L):
    f = L.q4g128_gemm_splitk
    args = [FAKE, 1, 256, FAKE, FAKE, FAKE, 16]
    assert f(*args, FAKE, 0, FAKE, 1 << 20, None) == q.Q4G128_EINVAL      # splits < 1
    assert f(*args, FAKE, 3, FAKE, 1 << 20, None) == q.Q4G128_EINVAL      # splits > K/128
    # more splits than 1024-k blocks pass the check (up to one per group);
    # they are launched only by the GPU tests.
    big = [FAKE, 1, 2048, FAKE, FAKE, FAKE, 16]
    assert f(*big, FAKE, 2, None, 1 << 20, None) == q.Q4G128_EINVAL       # no workspace
    assert f(*big, FAKE, 2, FAKE + 2, 1 << 20, None) == q.Q4G128_EINVAL   # misaligned
    assert f(*big, FAKE, 2, FAKE, 2 * 16 * 4 - 4, None) == q.Q4G128_EWORKSPACE
    assert f(FAKE, 1, 250, FAKE, FAKE, FAKE, 16, FAKE, 2, FAKE, 1 << 20, None) == q.Q4G128_EINVAL


def test_dequant_rejects(L):
    f = L.q4g128_dequant
    assert f(None, FAKE, FAKE, 256, 4, FAKE, None) == q.Q4G128_EINVAL
    assert f(FAKE, FAKE, FAKE, 200, 4, FAKE, None) == q.Q4G128_EINVAL
    assert f(FAKE, FAKE, FAKE, 256, 0, FAKE, None) == q.Q4G128_EINVAL
    assert f(FAKE, FAKE, FAKE, 256, 4, FAKE + 4, None) == q.Q4G128_EINVAL


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 128), dtype=torch.bfloat16)
    W = torch.zeros((4, 16), dtype=torch.int32)
    s = torch.zeros((4, 1), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        q.q4g128_gemm(x, W, s, s)


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "quantized_decode_q4g128_amd")
    banned = ("import oracle", "from oracle", "q4o_", "q4g128_oracle")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                for b in banned:
                    assert b not in text, (f, b)


def test_streamk_workspace_bytes(L):
    parts = 2 * 2048 * 128 * 4
    assert q.q4g128_streamk_workspace_bytes(5120, 34816) == (parts + 4 * 2176 + 255) // 256 * 256
    assert q.q4g128_streamk_workspace_bytes(1024, 1) == (parts + 4 + 255) // 256 * 256
    assert q.q4g128_streamk_workspace_bytes(5120 + 128, 16) == 0      # K not a multiple of 1024
    assert q.q4g128_streamk_workspace_bytes(1024, 0) == 0


def test_streamk_rejects(L):
    f = L.q4g128_gemm_streamk
    ok = [FAKE, 1, 2048, FAKE, FAKE, FAKE, 16, FAKE]
    need = q.q4g128_streamk_workspace_bytes(2048, 16)
    assert f(FAKE, 1, 2048 + 128, FAKE, FAKE, FAKE, 16, FAKE, FAKE, need, None) == q.Q4G128_EINVAL
    assert f(*ok, None, need, None) == q.Q4G128_EINVAL                   # no workspace
    assert f(*ok, FAKE + 16, need, None) == q.Q4G128_EINVAL              # not 256-byte aligned
    assert f(*ok, FAKE, need - 4, None) == q.Q4G128_EWORKSPACE
    assert f(FAKE, 1, 2048, FAKE, FAKE + 2, FAKE, 16, FAKE, FAKE, need, None) == q.Q4G128_EINVAL   # scale not 16-aligned
    assert f(FAKE, 9, 2048, FAKE, FAKE, FAKE, 16, FAKE, FAKE, need, None) == q.Q4G128_EINVAL   # stream-K: M <= 8


def test_quantize_rejects(L):
    f = L.q4g128_quantize
    ok = dict(w=FAKE, K=256, N=4, ncand=9, W=FAKE, s=FAKE, m=FAKE, e=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["w"], a["K"], a["N"], a["ncand"], a["W"], a["s"], a["m"], a["e"], None)

    for kw in (dict(w=None), dict(W=None), dict(s=None), dict(m=None), dict(K=200), dict(K=0), dict(N=0),
               dict(ncand=0), dict(ncand=17), dict(w=FAKE + 2), dict(W=FAKE + 4), dict(s=FAKE + 1),
               dict(e=FAKE + 4)):
        assert call(**kw) == q.Q4G128_EINVAL, kw


def test_epilogue_rejects(L):
    f = L.q4g128_gemm_swiglu
    need = q.q4g128_swiglu_workspace_bytes(1, 1024, 64)
    assert need == 64 * 4
    assert q.q4g128_swiglu_workspace_bytes(1, 1024, 63) == 0                      # odd N
    ok = [FAKE, 1, 1024, FAKE, FAKE, FAKE]
    assert f(*ok, 63, FAKE, FAKE, need, None) == q.Q4G128_EINVAL                 # odd N
    assert f(*ok, 64, None, FAKE, need, None) == q.Q4G128_EINVAL                 # no act
    assert f(*ok, 64, FAKE + 1, FAKE, need, None) == q.Q4G128_EINVAL             # act misaligned
    assert f(*ok, 64, FAKE, None, need, None) == q.Q4G128_EINVAL                 # no workspace
    assert f(*ok, 64, FAKE, FAKE, need - 4, None) == q.Q4G128_EWORKSPACE
    g = L.q4g128_gemm_rmsnorm
    base = [FAKE, 1, 1024, FAKE, FAKE, FAKE, 64]
    wsb = q.q4g128_rmsnorm_workspace_bytes(1, 64, 1)
    assert wsb == 256 + 64 * 4                                          # control block + partials
    assert q.q4g128_rmsnorm_workspace_bytes(2, 64, 3) == 256 + 3 * 2 * 64 * 4
    assert q.q4g128_rmsnorm_workspace_bytes(0, 64, 1) == 0
    assert g(*base, FAKE, FAKE, 1e-6, FAKE, FAKE, 1, FAKE, wsb - 256, None) == q.Q4G128_EWORKSPACE
    assert g(*base, None, FAKE, 1e-6, FAKE, FAKE, 1, FAKE, wsb, None) == q.Q4G128_EINVAL    # no residual
    assert g(*base, FAKE, None, 1e-6, FAKE, FAKE, 1, FAKE, wsb, None) == q.Q4G128_EINVAL    # no gamma
    assert g(*base, FAKE, FAKE, -1.0, FAKE, FAKE, 1, FAKE, wsb, None) == q.Q4G128_EINVAL    # eps < 0
    assert g(*base, FAKE, FAKE, float("nan"), FAKE, FAKE, 1, FAKE, wsb, None) == q.Q4G128_EINVAL
    # (x_out NULL is the residual-only form: a valid call, launched only by the GPU tests)
    assert g(*base, FAKE, FAKE, 1e-6, FAKE, FAKE, 0, FAKE, wsb, None) == q.Q4G128_EINVAL    # splits 0
    assert g(*base, FAKE, FAKE, 1e-6, FAKE, FAKE, 9, FAKE, 10 ** 6, None) == q.Q4G128_EINVAL   # > K/128
    assert g(*base, FAKE, FAKE, 1e-6, FAKE, FAKE, 1, FAKE, wsb - 4, None) == q.Q4G128_EWORKSPACE


def test_splitk_noalloc_rejects_before_launch(L):
    f = L.q4g128_gemm_splitk_noalloc
    args = [FAKE, 1, 256, FAKE, FAKE, FAKE, 16, FAKE]
    assert f(*args, 0, None) == q.Q4G128_EINVAL                           # splits < 1
    assert f(*args, 3, None) == q.Q4G128_EINVAL                           # splits > K/128
    assert f(None, 1, 256, FAKE, FAKE, FAKE, 16, FAKE, 2, None) == q.Q4G128_EINVAL
    # 136 splits x 16 rows x 5120 columns x 4 bytes = 44.6 MB > the 8 MiB scratch
    assert f(FAKE, 16, 17408, FAKE, FAKE, FAKE, 5120, FAKE, 136, None) == q.Q4G128_EWORKSPACE
    assert b"exceeds the library scratch" in L.q4g128_last_error()


def test_prenorm_workspace_and_rejects(L):
    assert q.q4g128_prenorm_workspace_bytes(1, 5120, 12288) == 10240
    assert q.q4g128_prenorm_workspace_bytes(3, 128, 2, True) == 768 + q.q4g128_swiglu_workspace_bytes(3, 128, 2)
    for bad in ((0, 1024, 16, 0), (17, 1024, 16, 0), (1, 100, 16, 0), (1, 1024, 0, 0), (1, 1024, 3, 1)):
        assert q.q4g128_prenorm_workspace_bytes(*bad) == 0
    f, g = L.q4g128_gemm_prenorm, L.q4g128_gemm_swiglu_prenorm
    need = q.q4g128_prenorm_workspace_bytes(1, 1024, 64)

    def call(fn, h=FAKE, gamma=FAKE, eps=1e-6, M=1, K=1024, W=FAKE, s=FAKE, m=FAKE, N=64, out=FAKE, ws=FAKE,
             nb=None):
        return fn(h, gamma, eps, M, K, W, s, m, N, out, ws, need if nb is None else nb, None)

    for fn in (f, g):
        for kw in (dict(h=None), dict(gamma=None), dict(W=None), dict(s=None), dict(m=None), dict(out=None),
                   dict(h=FAKE + 2), dict(gamma=FAKE + 1), dict(W=FAKE + 4), dict(eps=-1.0),
                   dict(eps=float("nan")), dict(M=0), dict(M=17), dict(K=100), dict(N=0), dict(ws=None),
                   dict(ws=FAKE + 16)):
            assert call(fn, **kw) == q.Q4G128_EINVAL, (fn, kw)
    assert call(f, nb=need - 4) == q.Q4G128_EWORKSPACE
    assert call(g, N=63) == q.Q4G128_EINVAL                                  # odd N
    assert call(g, nb=q.q4g128_prenorm_workspace_bytes(1, 1024, 64, True) - 4) == q.Q4G128_EWORKSPACE


def test_rmsnorm_residual_only_arguments(L):
    g = L.q4g128_gemm_rmsnorm
    base = [FAKE, 1, 1024, FAKE, FAKE, FAKE, 64]
    wsb = q.q4g128_rmsnorm_workspace_bytes(1, 64, 1)
    # x_out NULL: gamma and eps are not read (so bad values do not reject) ...
    assert g(*base, None, None, -1.0, FAKE, None, 1, FAKE, wsb, None) == q.Q4G128_EINVAL   # ... residual still
    assert g(*base, FAKE + 2, None, -1.0, FAKE, None, 1, FAKE, wsb, None) == q.Q4G128_EINVAL
    assert g(*base, FAKE, None, -1.0, FAKE, None, 1, FAKE, wsb - 4, None) == q.Q4G128_EWORKSPACE

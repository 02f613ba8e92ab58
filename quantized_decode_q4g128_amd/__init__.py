"""Python binding of libq4g128.so: the int4-g128 weight-streaming product on
AMD MI355X (gfx950).

Argument marshalling only.  Every step of the product runs in the library's
HIP kernels; PyTorch supplies device memory and the stream.  The functions
carry the C ABI's names (include/q4g128.h) and take torch tensors:

    x      [M][K]    bf16 (or int16/uint16 holding bf16 bit patterns), 1 <= M <= 16
    W      [N][K/8]  int32/uint32 packed codes, low nibble first
    scale  [N][K/128] bf16 (or 16-bit bit patterns)
    min    [N][K/128] bf16 (or 16-bit bit patterns)
    y      [M][N]    float32

There is no CPU fallback: if the library is missing, or a tensor is not on a
GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq4g128.so")

Q4G128_OK, Q4G128_EINVAL, Q4G128_EWORKSPACE, Q4G128_EHIP = 0, 1, 2, 3
GROUP = 128
MAX_M = 16

_lib = None


class Q4G128Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(what)


def lib() -> ctypes.CDLL:
    """The loaded libq4g128.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Q4G128Error(-1, f"libq4g128.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.q4g128_gemm.argtypes = [vp, ci, ci, vp, vp, vp, ci, vp, vp]
        L.q4g128_gemm.restype = ci
        L.q4g128_gemm_splitk.argtypes = [vp, ci, ci, vp, vp, vp, ci, vp, ci, vp, sz, vp]
        L.q4g128_gemm_splitk.restype = ci
        L.q4g128_gemm_splitk_noalloc.argtypes = [vp, ci, ci, vp, vp, vp, ci, vp, ci, vp]
        L.q4g128_gemm_splitk_noalloc.restype = ci
        L.q4g128_gemm_streamk.argtypes = [vp, ci, ci, vp, vp, vp, ci, vp, vp, sz, vp]
        L.q4g128_gemm_streamk.restype = ci
        L.q4g128_streamk_workspace_bytes.argtypes = [ci, ci]
        L.q4g128_streamk_workspace_bytes.restype = sz
        L.q4g128_dequant.argtypes = [vp, vp, vp, ci, ci, vp, vp]
        L.q4g128_dequant.restype = ci
        L.q4g128_swiglu_workspace_bytes.argtypes = [ci, ci, ci]
        L.q4g128_swiglu_workspace_bytes.restype = sz
        L.q4g128_gemm_swiglu.argtypes = [vp, ci, ci, vp, vp, vp, ci, vp, vp, sz, vp]
        L.q4g128_gemm_swiglu.restype = ci
        L.q4g128_gemm_rmsnorm.argtypes = [vp, ci, ci, vp, vp, vp, ci, vp, vp, ctypes.c_float, vp, vp, ci, vp, sz,
                                          vp]
        L.q4g128_gemm_rmsnorm.restype = ci
        L.q4g128_quantize.argtypes = [vp, ci, ci, ci, vp, vp, vp, vp, vp]
        L.q4g128_quantize.restype = ci
        L.q4g128_splitk_workspace_bytes.argtypes = [ci, ci, ci]
        L.q4g128_splitk_workspace_bytes.restype = sz
        L.q4g128_rmsnorm_workspace_bytes.argtypes = [ci, ci, ci]
        L.q4g128_rmsnorm_workspace_bytes.restype = sz
        L.q4g128_prenorm_workspace_bytes.argtypes = [ci, ci, ci, ci]
        L.q4g128_prenorm_workspace_bytes.restype = sz
        L.q4g128_gemm_prenorm.argtypes = [vp, vp, ctypes.c_float, ci, ci, vp, vp, vp, ci, vp, vp, sz, vp]
        L.q4g128_gemm_prenorm.restype = ci
        L.q4g128_gemm_swiglu_prenorm.argtypes = [vp, vp, ctypes.c_float, ci, ci, vp, vp, vp, ci, vp, vp, sz, vp]
        L.q4g128_gemm_swiglu_prenorm.restype = ci
        L.q4g128_gemm_parts.argtypes = [ci, ci]
        L.q4g128_gemm_parts.restype = ci
        L.q4g128_splitk_default_splits.argtypes = [ci, ci]
        L.q4g128_splitk_default_splits.restype = ci
        L.q4g128_status_string.argtypes = [ci]
        L.q4g128_status_string.restype = ctypes.c_char_p
        L.q4g128_last_error.argtypes = []
        L.q4g128_last_error.restype = ctypes.c_char_p
        L.q4g128_abi_version.argtypes = []
        L.q4g128_abi_version.restype = ci
        _lib = L
    return _lib


def q4g128_abi_version() -> int:
    return int(lib().q4g128_abi_version())


def q4g128_status_string(status: int) -> str:
    return lib().q4g128_status_string(int(status)).decode()


def q4g128_last_error() -> str:
    return lib().q4g128_last_error().decode()


def q4g128_splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    return int(lib().q4g128_splitk_workspace_bytes(int(M), int(N), int(splits)))


def q4g128_rmsnorm_workspace_bytes(M: int, N: int, splits: int) -> int:
    return int(lib().q4g128_rmsnorm_workspace_bytes(int(M), int(N), int(splits)))


def q4g128_rmsnorm_workspace(M: int, N: int, splits: int, device) -> torch.Tensor:
    """A zero-filled workspace for q4g128_gemm_rmsnorm on (M, N, splits);
    reusable by later calls of that size or smaller (they leave its control
    block zero) as long as nothing else writes it."""
    nbytes = q4g128_rmsnorm_workspace_bytes(M, N, splits)
    if nbytes == 0:
        raise ValueError(f"invalid rmsnorm workspace request M={M} N={N} splits={splits}")
    return torch.zeros((nbytes // 4,), dtype=torch.float32, device=device)


def q4g128_splitk_default_splits(K: int, N: int) -> int:
    return int(lib().q4g128_splitk_default_splits(int(K), int(N)))


def q4g128_gemm_parts(K: int, N: int) -> int:
    """Split count whose q4g128_gemm_splitk bits equal q4g128_gemm's (1: no cut)."""
    return int(lib().q4g128_gemm_parts(int(K), int(N)))


# ---- marshalling helpers -----------------------------------------------------

_HALF = (torch.bfloat16, torch.int16, torch.uint16)
_WORD = (torch.int32, torch.uint32)


def _dev(t: torch.Tensor, name: str, dtypes, ndim: int = 2) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device}); there is no CPU path")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-D tensor (got shape {tuple(t.shape)})")
    return t


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != Q4G128_OK:
        detail = q4g128_last_error() if status == Q4G128_EHIP else ""
        raise Q4G128Error(status, f"{what}: {q4g128_status_string(status)} {detail}".strip())


def _operands(x, W, scale, min):
    x = _dev(x, "x", _HALF)
    W = _dev(W, "W", _WORD)
    scale = _dev(scale, "scale", _HALF)
    min = _dev(min, "min", _HALF)
    M, K = x.shape
    N = W.shape[0]
    if W.shape[1] * 8 != K:
        raise ValueError(f"W has {W.shape[1]} words per column; x has K={K} (needs K/8)")
    if K % GROUP or tuple(scale.shape) != (N, K // GROUP) or tuple(min.shape) != (N, K // GROUP):
        raise ValueError(f"scale/min must be [N][K/128] = {(N, K // GROUP)}")
    for t in (W, scale, min):
        if t.device != x.device:
            raise ValueError("all operands must be on the same device")
    return x, W, scale, min, M, K, N


def _out(y, M, N, device):
    if y is None:
        return torch.empty((M, N), dtype=torch.float32, device=device)
    y = _dev(y, "y", (torch.float32,))
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be [M][N] = {(M, N)}")
    return y


# ---- entry points ------------------------------------------------------------

def q4g128_gemm(x, W, scale, min, y=None, stream=None) -> torch.Tensor:
    """y[M][N] = x . dequant(W), K not split (one launch)."""
    x, W, scale, min, M, K, N = _operands(x, W, scale, min)
    y = _out(y, M, N, x.device)
    st = lib().q4g128_gemm(x.data_ptr(), M, K, W.data_ptr(), scale.data_ptr(), min.data_ptr(), N,
                           y.data_ptr(), _stream(stream, x.device))
    _check(st, "q4g128_gemm")
    return y


def q4g128_gemm_splitk(x, W, scale, min, splits=None, workspace=None, y=None, stream=None) -> torch.Tensor:
    """y = x . dequant(W) with K cut into `splits` group-aligned ranges
    (default: q4g128_splitk_default_splits(K, N)); partial sums go to
    `workspace` (allocated here if not given) and are summed in split order."""
    x, W, scale, min, M, K, N = _operands(x, W, scale, min)
    y = _out(y, M, N, x.device)
    if splits is None:
        splits = q4g128_splitk_default_splits(K, N)
    need = q4g128_splitk_workspace_bytes(M, N, splits) if splits >= 1 else 0
    if workspace is None:
        workspace = torch.empty((max(need, 4) // 4,), dtype=torch.float32, device=x.device)
    workspace = _dev(workspace, "workspace", (torch.float32,), ndim=workspace.dim())
    ws_bytes = workspace.numel() * 4
    st = lib().q4g128_gemm_splitk(x.data_ptr(), M, K, W.data_ptr(), scale.data_ptr(), min.data_ptr(), N,
                                  y.data_ptr(), int(splits), workspace.data_ptr(), ws_bytes,
                                  _stream(stream, x.device))
    _check(st, "q4g128_gemm_splitk")
    return y


def q4g128_gemm_splitk_noalloc(x, W, scale, min, y, splits=None, stream=None) -> torch.Tensor:
    """q4g128_gemm_splitk with the partial sums in the library's own device
    scratch (8 MiB per GPU): the call allocates nothing, so y must be given.
    Calls overlapping on one GPU race on that scratch."""
    x, W, scale, min, M, K, N = _operands(x, W, scale, min)
    if y is None:
        raise ValueError("y must be given: q4g128_gemm_splitk_noalloc allocates nothing")
    y = _out(y, M, N, x.device)
    if splits is None:
        splits = q4g128_splitk_default_splits(K, N)
    st = lib().q4g128_gemm_splitk_noalloc(x.data_ptr(), M, K, W.data_ptr(), scale.data_ptr(), min.data_ptr(), N,
                                          y.data_ptr(), int(splits), _stream(stream, x.device))
    _check(st, "q4g128_gemm_splitk_noalloc")
    return y


def q4g128_streamk_workspace_bytes(K: int, N: int) -> int:
    return int(lib().q4g128_streamk_workspace_bytes(int(K), int(N)))


def q4g128_streamk_workspace(K: int, N: int, device) -> torch.Tensor:
    """A zero-filled workspace for q4g128_gemm_streamk on (K, N); reusable by
    successive calls (each call leaves it zero-filled), one call at a time."""
    nbytes = q4g128_streamk_workspace_bytes(K, N)
    if nbytes == 0:
        raise ValueError(f"stream-K does not support K={K}, N={N} (K must be a multiple of 1024)")
    return torch.zeros((nbytes // 4,), dtype=torch.int32, device=device)


def q4g128_gemm_streamk(x, W, scale, min, workspace=None, y=None, stream=None) -> torch.Tensor:
    """y = x . dequant(W) with the work spread evenly over the compute units.
    `workspace` must come from q4g128_streamk_workspace (zero-filled) and must
    not be in use by another call in flight; one is allocated if not given."""
    x, W, scale, min, M, K, N = _operands(x, W, scale, min)
    y = _out(y, M, N, x.device)
    if workspace is None:
        workspace = q4g128_streamk_workspace(K, N, x.device)
    if workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the operands' device")
    st = lib().q4g128_gemm_streamk(x.data_ptr(), M, K, W.data_ptr(), scale.data_ptr(), min.data_ptr(), N,
                                   y.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(stream, x.device))
    _check(st, "q4g128_gemm_streamk")
    return y


def q4g128_dequant(W, scale, min, out=None, stream=None) -> torch.Tensor:
    """Decoded weights fp32 [N][K], w = fp32(q*s + m) rounded once."""
    W = _dev(W, "W", _WORD)
    scale = _dev(scale, "scale", _HALF)
    min = _dev(min, "min", _HALF)
    N, K = W.shape[0], W.shape[1] * 8
    if tuple(scale.shape) != (N, K // GROUP) or tuple(min.shape) != (N, K // GROUP):
        raise ValueError(f"scale/min must be [N][K/128] = {(N, K // GROUP)}")
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=W.device)
    out = _dev(out, "out", (torch.float32,))
    if tuple(out.shape) != (N, K):
        raise ValueError(f"out must be [N][K] = {(N, K)}")
    st = lib().q4g128_dequant(W.data_ptr(), scale.data_ptr(), min.data_ptr(), K, N, out.data_ptr(),
                              _stream(stream, W.device))
    _check(st, "q4g128_dequant")
    return out


def q4g128_swiglu_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().q4g128_swiglu_workspace_bytes(int(M), int(K), int(N)))


def _half_out(t, name, shape, device):
    if t is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=device)
    t = _dev(t, name, _HALF)
    if tuple(t.shape) != shape or t.device != device:
        raise ValueError(f"{name} must be {shape} on {device}")
    return t


def _workspace(ws, need, device):
    if ws is None:
        ws = torch.empty((max(need, 4) // 4,), dtype=torch.float32, device=device)
    ws = _dev(ws, "workspace", (torch.float32,), ndim=ws.dim())
    if ws.device != device:
        raise ValueError("workspace must be on the operands' device")
    return ws


def q4g128_gemm_swiglu(x, W, scale, min, act=None, workspace=None, stream=None) -> torch.Tensor:
    """act [M][N/2] bf16 = silu(gate) * up of the fused gate/up product
    (gate = output columns 0..N/2-1, up = the rest)."""
    x, W, scale, min, M, K, N = _operands(x, W, scale, min)
    if N % 2:
        raise ValueError(f"N={N} must be even (gate and up halves)")
    act = _half_out(act, "act", (M, N // 2), x.device)
    workspace = _workspace(workspace, q4g128_swiglu_workspace_bytes(M, K, N), x.device)
    st = lib().q4g128_gemm_swiglu(x.data_ptr(), M, K, W.data_ptr(), scale.data_ptr(), min.data_ptr(), N,
                                  act.data_ptr(), workspace.data_ptr(), workspace.numel() * 4,
                                  _stream(stream, x.device))
    _check(st, "q4g128_gemm_swiglu")
    return act


def q4g128_gemm_rmsnorm(x, W, scale, min, residual, gamma, eps: float = 1e-6, splits=None, h=None, x_out=None,
                        workspace=None, stream=None, norm: bool = True):
    """(h, x_out): h = residual + x . dequant(W) (fp32 [M][N]; pass h=residual
    to update it in place), x_out = bf16(h / sqrt(mean(h^2) + eps) * gamma),
    the split-K partials (default split count) summed inside the norm.
    norm=False: the residual add alone, returns (h, None) (gamma unused: the
    next product normalises h itself, q4g128_gemm_prenorm).
    A given `workspace` must come from q4g128_rmsnorm_workspace (its first
    256 bytes zero; every call leaves them so) and must not be written by
    other calls in between."""
    x, W, scale, min, M, K, N = _operands(x, W, scale, min)
    residual = _dev(residual, "residual", (torch.float32,))
    if tuple(residual.shape) != (M, N) or residual.device != x.device:
        raise ValueError(f"residual must be [M][N] = {(M, N)} on the operands' device")
    if norm:
        gamma = _dev(gamma, "gamma", _HALF, ndim=1)
        if tuple(gamma.shape) != (N,) or gamma.device != x.device:
            raise ValueError(f"gamma must be [N] = ({N},) on the operands' device")
    h = _out(h, M, N, x.device)
    x_out = _half_out(x_out, "x_out", (M, N), x.device) if norm else None
    if splits is None:
        splits = q4g128_splitk_default_splits(K, N)
    if workspace is None and splits >= 1:
        workspace = q4g128_rmsnorm_workspace(M, N, splits, x.device)
    workspace = _workspace(workspace, 0, x.device)
    st = lib().q4g128_gemm_rmsnorm(x.data_ptr(), M, K, W.data_ptr(), scale.data_ptr(), min.data_ptr(), N,
                                   residual.data_ptr(), gamma.data_ptr() if norm else None, float(eps), h.data_ptr(),
                                   x_out.data_ptr() if norm else None, int(splits), workspace.data_ptr(),
                                   workspace.numel() * 4, _stream(stream, x.device))
    _check(st, "q4g128_gemm_rmsnorm")
    return h, x_out


def q4g128_prenorm_workspace_bytes(M: int, K: int, N: int, swiglu: bool = False) -> int:
    return int(lib().q4g128_prenorm_workspace_bytes(int(M), int(K), int(N), 1 if swiglu else 0))


def _prenorm_operands(h, gamma, W, scale, min):
    h = _dev(h, "h", (torch.float32,))
    gamma = _dev(gamma, "gamma", _HALF, ndim=1)
    W = _dev(W, "W", _WORD)
    scale = _dev(scale, "scale", _HALF)
    min = _dev(min, "min", _HALF)
    M, K = h.shape
    N = W.shape[0]
    if W.shape[1] * 8 != K or tuple(gamma.shape) != (K,):
        raise ValueError(f"W must be [N][K/8] and gamma [K] for h of K={K}")
    if K % GROUP or tuple(scale.shape) != (N, K // GROUP) or tuple(min.shape) != (N, K // GROUP):
        raise ValueError(f"scale/min must be [N][K/128] = {(N, K // GROUP)}")
    for t in (gamma, W, scale, min):
        if t.device != h.device:
            raise ValueError("all operands must be on the same device")
    return h, gamma, W, scale, min, M, K, N


def _ws256(ws, need, device):
    """A 256-byte aligned workspace of at least `need` bytes."""
    if ws is None:
        ws = torch.empty((max(need, 256) // 4,), dtype=torch.float32, device=device)
    ws = _workspace(ws, need, device)
    if ws.data_ptr() % 256:
        raise ValueError("workspace must be 256-byte aligned")
    return ws


def q4g128_gemm_prenorm(h, gamma, W, scale, min, eps: float = 1e-6, y=None, workspace=None,
                        stream=None) -> torch.Tensor:
    """y = x . dequant(W) with x = bf16(h / sqrt(mean(h^2) + eps) * gamma)
    made from fp32 rows h inside the product (the x_out q4g128_gemm_rmsnorm
    would give for h, bit for bit)."""
    h, gamma, W, scale, min, M, K, N = _prenorm_operands(h, gamma, W, scale, min)
    y = _out(y, M, N, h.device)
    workspace = _ws256(workspace, q4g128_prenorm_workspace_bytes(M, K, N), h.device)
    st = lib().q4g128_gemm_prenorm(h.data_ptr(), gamma.data_ptr(), float(eps), M, K, W.data_ptr(), scale.data_ptr(),
                                   min.data_ptr(), N, y.data_ptr(), workspace.data_ptr(), workspace.numel() * 4,
                                   _stream(stream, h.device))
    _check(st, "q4g128_gemm_prenorm")
    return y


def q4g128_gemm_swiglu_prenorm(h, gamma, W, scale, min, eps: float = 1e-6, act=None, workspace=None,
                               stream=None) -> torch.Tensor:
    """q4g128_gemm_swiglu on x = the normalised h (as q4g128_gemm_prenorm)."""
    h, gamma, W, scale, min, M, K, N = _prenorm_operands(h, gamma, W, scale, min)
    if N % 2:
        raise ValueError(f"N={N} must be even (gate and up halves)")
    act = _half_out(act, "act", (M, N // 2), h.device)
    workspace = _ws256(workspace, q4g128_prenorm_workspace_bytes(M, K, N, True), h.device)
    st = lib().q4g128_gemm_swiglu_prenorm(h.data_ptr(), gamma.data_ptr(), float(eps), M, K, W.data_ptr(),
                                          scale.data_ptr(), min.data_ptr(), N, act.data_ptr(), workspace.data_ptr(),
                                          workspace.numel() * 4, _stream(stream, h.device))
    _check(st, "q4g128_gemm_swiglu_prenorm")
    return act


def q4g128_quantize(w, ncand: int = 9, W=None, scale=None, min=None, err=None, stream=None):
    """bf16 weights w [N][K] -> (W [N][K/8] int32, scale [N][K/128] int16
    bf16 bits, min [N][K/128] int16 bf16 bits, err [N][K/128] float64): the
    per-group range search over ncand x ncand clipped ranges (ncand = 1 is
    round-to-nearest).  A group holding a NaN or infinity comes back with
    err NaN and zero codes, scale and min."""
    w = _dev(w, "w", _HALF)
    N, K = w.shape
    if K % GROUP:
        raise ValueError(f"K={K} must be a multiple of {GROUP}")
    G = K // GROUP
    dev = w.device

    def out(t, name, shape, dtypes, dtype):
        if t is None:
            return torch.empty(shape, dtype=dtype, device=dev)
        t = _dev(t, name, dtypes)
        if tuple(t.shape) != shape or t.device != dev:
            raise ValueError(f"{name} must be {shape} on {dev}")
        return t

    W = out(W, "W", (N, K // 8), _WORD, torch.int32)
    scale = out(scale, "scale", (N, G), _HALF, torch.int16)
    min = out(min, "min", (N, G), _HALF, torch.int16)
    err = out(err, "err", (N, G), (torch.float64,), torch.float64)
    st = lib().q4g128_quantize(w.data_ptr(), K, N, int(ncand), W.data_ptr(), scale.data_ptr(), min.data_ptr(),
                               err.data_ptr(), _stream(stream, dev))
    _check(st, "q4g128_quantize")
    return W, scale, min, err


__all__ = ["q4g128_gemm", "q4g128_quantize", "q4g128_gemm_swiglu", "q4g128_swiglu_workspace_bytes",
           "q4g128_gemm_rmsnorm", "q4g128_rmsnorm_workspace", "q4g128_rmsnorm_workspace_bytes",
           "q4g128_gemm_prenorm", "q4g128_gemm_swiglu_prenorm", "q4g128_prenorm_workspace_bytes",
           "q4g128_gemm_splitk", "q4g128_gemm_splitk_noalloc", "q4g128_gemm_streamk", "q4g128_streamk_workspace",
           "q4g128_streamk_workspace_bytes", "q4g128_dequant", "q4g128_splitk_workspace_bytes",
           "q4g128_splitk_default_splits", "q4g128_gemm_parts", "q4g128_status_string", "q4g128_last_error",
           "q4g128_abi_version", "Q4G128Error", "lib", "LIB_PATH"]

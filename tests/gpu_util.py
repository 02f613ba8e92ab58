"""Helpers for the GPU tests: move seeded synthetic cases to the device and
compare results with the oracle."""
import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")


def dev_x(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV)


def dev_weights(wt):
    W = torch.from_numpy(np.ascontiguousarray(wt.W).view(np.int32)).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(wt.scale).view(np.int16)).to(DEV)
    m = torch.from_numpy(np.ascontiguousarray(wt.mn).view(np.int16)).to(DEV)
    return W, s, m


def host_f32(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize(DEV)
    return t.detach().cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_within_tolerance(y_gpu, y_ref, a_ref, what=""):
    ok = oracle.within_tolerance(y_gpu, y_ref, a_ref)
    if not ok.all():
        bad = np.argwhere(~ok)
        m, n = bad[0]
        err = abs(float(y_gpu[m, n]) - y_ref[m, n])
        raise AssertionError(f"{what}: {len(bad)} outputs outside |y-y_ref| <= 1e-3*a + 1e-6; "
                             f"first at (m={m}, n={n}): gpu={y_gpu[m, n]!r} ref={y_ref[m, n]!r} "
                             f"a={a_ref[m, n]!r} err={err:.3e}")
    # Report the worst margin so regressions in accuracy are visible in logs.
    return float(np.max(np.abs(y_gpu - y_ref) / (1e-3 * a_ref + 1e-6)))

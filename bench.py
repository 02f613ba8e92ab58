"""Benchmark of the int4-g128 weight-streaming product on one MI355X.

One step = one call of the product on the decode gate/up projection
(M=1, K=5120, N=34816: two 17408-wide projections fused along N) with int4
codes, bf16 scale and minimum per 128 weights, bf16 x, fp32 accumulation and
output.  Inputs are synthetic (seeded; distributions of the quantised
matrices and activations the pages measure on) and resident in HBM before the
timed region.  Each step reads a different copy of the weights, cycling over
>= 1.2 GB of copies, so no step is served from the 256 MB last-level cache.

Reported: algorithmic bytes per step / time as GB/s (value), the same at M=7
(speculative verify) and the verify/decode time ratio, the dominant kernel's
roofline (HIP-event kernel durations; bytes from the format: K*N/2 codes +
4*N*K/128 scale/min + 2*M*K x + 4*M*N y), and the fp64 CPU oracle's rate on
the host as a baseline.  A result that fails parity against the oracle is not
reported (value null).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E peak, 8 TB/s
ROTATE_BYTES = 1.2e9            # > 4x the 256 MB last-level cache
METRIC = "achieved HBM GB/s (% of MI355X peak) for int4-g128 GEMV at M=1 and M=7"


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="bounded CPU time budget for the oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


class Rotation:
    """R device copies of one weight set plus one x; call i uses copy i % R."""

    def __init__(self, case, torch, q):
        self.torch, self.q = torch, q
        wt = case.weights
        self.M, self.K, self.N = case.M, case.K, case.N
        self.bytes = synth.algorithmic_bytes(self.M, self.K, self.N)
        self.R = max(2, math.ceil(ROTATE_BYTES / self.bytes))
        dev = torch.device("cuda:0")
        W = torch.from_numpy(wt.W.view(np.int32)).to(dev)
        s = torch.from_numpy(wt.scale.view(np.int16)).to(dev)
        m = torch.from_numpy(wt.mn.view(np.int16)).to(dev)
        self.sets = [(W, s, m)] + [(W.clone(), s.clone(), m.clone()) for _ in range(self.R - 1)]
        self.x = torch.from_numpy(case.x.view(np.int16)).to(dev)
        self.y = torch.empty((self.M, self.N), dtype=torch.float32, device=dev)

    def call(self, i, stream):
        W, s, m = self.sets[i % self.R]
        self.q.q4g128_gemm(self.x, W, s, m, y=self.y, stream=stream)

    def timed(self, steps, warmup):
        """Milliseconds for `steps` back-to-back calls, bracketed by HIP events
        recorded on the stream the kernels run on (events around every single
        launch would add their own overhead to each call)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        for i in range(warmup):
            self.call(i, stream)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(steps):
            self.call(warmup + i, stream)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)


def cpu_baseline(case, budget_s):
    import oracle
    orc = oracle.load()
    wt = case.weights
    t0 = time.perf_counter()
    y, a = orc.gemm(case.x, wt.W, wt.scale, wt.mn)
    reps = 1
    while time.perf_counter() - t0 < budget_s and reps < 1000:
        orc.gemm(case.x, wt.W, wt.scale, wt.mn)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    B = synth.algorithmic_bytes(case.M, case.K, case.N)
    return {"value": B / dt / 1e9, "unit": "GB/s", "cores": orc.max_threads(), "kind": "oracle",
            "sample": f"{reps} full fp64 oracle calls on the same M={case.M} K={case.K} N={case.N} "
                      f"input ({dt * 1e3:.1f} ms per call)"}, (y, a)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_decode_q4g128_amd as q
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    dec_case = synth.make_case("gateup")
    ver_case = synth.make_case("verify", 7)
    dec = Rotation(dec_case, torch, q)
    ver = Rotation(ver_case, torch, q)

    # Parity gate on the exact launches that get timed (first rotation set).
    stream = torch.cuda.current_stream()
    dec.call(0, stream)
    y_dec = dec.y.cpu().numpy()
    ver.call(0, stream)
    y_ver = ver.y.cpu().numpy()

    cpu = None
    import oracle
    if not args.no_cpu_baseline:
        cpu, (yr, ar) = cpu_baseline(dec_case, args.cpu_seconds)
    else:
        yr, ar = oracle.load().gemm(dec_case.x, dec_case.weights.W, dec_case.weights.scale, dec_case.weights.mn)
    ok_dec = bool(oracle.within_tolerance(y_dec, yr, ar).all())
    yv, av = oracle.load().gemm(ver_case.x, ver_case.weights.W, ver_case.weights.scale, ver_case.weights.mn)
    ok_ver = bool(oracle.within_tolerance(y_ver, yv, av).all())

    wall_d = dec.timed(args.steps, args.warmup)
    wall_v = ver.timed(args.steps, args.warmup)
    ms_step = wall_d / args.steps
    t_dec = wall_d * 1e-3 / args.steps            # s per launch (back to back)
    t_ver = wall_v * 1e-3 / args.steps
    gbps = dec.bytes * args.steps / (wall_d * 1e-3) / 1e9
    achieved = dec.bytes / t_dec / 1e9
    ver_gbps = ver.bytes / t_ver / 1e9

    line = {
        "metric": METRIC,
        "value": round(gbps, 1) if ok_dec else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode gate/up projection, int4-g128, M=1 K=5120 N=34816",
                   "M": 1, "K": 5120, "N": 34816, "bytes_per_step": dec.bytes,
                   "weight_copies_rotated": dec.R, "accumulate": "fp32"},
        "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2) if ok_dec else None,
        "parity": {"decode_M1": "pass" if ok_dec else "FAIL", "verify_M7": "pass" if ok_ver else "FAIL"},
        "verify_M7": {"GBps": round(ver_gbps, 1) if ok_ver else None, "us_per_call": round(t_ver * 1e6, 3),
                      "bytes_per_call": ver.bytes,
                      "time_ratio_vs_M1": round(t_ver / t_dec, 4) if ok_ver and ok_dec else None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "kernel": "gemv_q4g128<1>", "us_per_launch": round(t_dec * 1e6, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

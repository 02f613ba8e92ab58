"""Benchmark of the int4-g128 weight-streaming product on one MI355X.

One step = one call of the product on the decode gate/up projection
(M=1, K=5120, N=34816: two 17408-wide projections fused along N) with int4
codes, bf16 scale and minimum per 128 weights, bf16 x, fp32 accumulation and
output.  Inputs are synthetic (seeded; distributions of the quantised
matrices and activations the pages measure on) and resident in HBM before the
timed region.  Each step reads a different copy of the weights, cycling over
>= 1.2 GB of copies, so no step is served from the 256 MB last-level cache.

Reported: algorithmic bytes per step / time as GB/s (value), the same at M=7
(speculative verify) and the verify/decode time ratio, the down projection
(split-K) and the full synthetic decode-step stream (257 launches, 12.7 GB)
as extra fields, the fused epilogues (gate/up + SwiGLU, down + residual-add
RMSNorm) alone and chained through a 64-layer decode step, eager and as a
HIP graph, the quantizer producing the format (the gate/up matrix from
bf16, 9 x 9 range search, fp64) as an extra field with its own fp64 ALU
roofline, the dominant kernel's
roofline (HIP-event kernel durations; bytes from the format: K*N/2 codes +
4*N*K/128 scale/min + 2*M*K x + 4*M*N y), and the fp64 CPU oracle's rate on
the host as a baseline, and beside the roofline what a pure read of the same
codes reaches on this GPU in the product's access pattern and contiguously
(libq4g128_probe.so).  The oracle runs only in the CPU leg (cpu_baseline),
after the GPU timing; it also computes the parity references, and a result
that fails parity against them is not reported (value null).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

HBM traffic of the dominant kernel comes from two rocprofv3 counter runs
(FETCH_SIZE, then WRITE_SIZE) of `--pmc-workload`, turned into a summary by
`--pmc-summarize`; the summary is keyed by a hash of the kernel sources and
ignored once they change:

    rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o run --output-format csv -- python3 bench.py --pmc-workload
    rocprofv3 --pmc WRITE_SIZE -d OUT/write -o run --output-format csv -- python3 bench.py --pmc-workload
    python3 bench.py --pmc-summarize OUT/fetch OUT/write profiles/gemv_q4g128_gateup_pmc.txt
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
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
PEAK_FP64_TFLOPS = 78.6         # MI355X fp64 vector peak
ROTATE_BYTES = 1.2e9            # > 4x the 256 MB last-level cache
WARM_S = 0.2                    # untimed launches before every timed leg, seconds
METRIC = "achieved HBM GB/s (% of MI355X peak) for int4-g128 GEMV at M=1 and M=7"
KERNEL = "gemv_q4g128_lds"      # the kernel of the decode gate/up launch (all of its time)
PMC_SUMMARY = os.path.join(ROOT, "profiles", "gemv_q4g128_gateup_pmc.txt")
TRACE_SUMMARY = os.path.join(ROOT, "profiles", "gemv_q4g128_gateup_kernel_trace.txt")
DIST_CALLS = 1300               # per-launch distribution: at least this many launches (100 passes over 13 copies)
COPY_BYTES = 256 << 20          # calibration copy for the traffic counters
PMC_LAUNCHES = 24


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="bounded CPU time budget for the oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-stream", action="store_true", help="skip the 12.7 GB decode-step stream")
    p.add_argument("--no-verify", action="store_true", help="skip the M=7 verify step (profiling decode alone)")
    p.add_argument("--no-down", action="store_true", help="skip the down projection")
    p.add_argument("--no-quantize", action="store_true", help="skip the quantizer measurement")
    p.add_argument("--no-epilogues", action="store_true", help="skip the fused-epilogue measurements")
    p.add_argument("--no-read-ceiling", action="store_true", help="skip the pure-read probes")
    p.add_argument("--stream-only", action="store_true",
                   help="run only the decode-step stream (for a kernel trace of it) and print its fields")
    p.add_argument("--pmc-workload", action="store_true",
                   help="run the counter workload (a known-size copy, then decode launches) and exit")
    p.add_argument("--pmc-summarize", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"),
                   help="turn two rocprofv3 counter runs of --pmc-workload into a traffic summary")
    p.add_argument("--pmc-shape", nargs=2, type=int, metavar=("K", "N"), default=None,
                   help="the counter workload's product shape at M=1 (default: the decode gate/up projection, "
                        "K=5120 N=34816; another shape draws seeded random weights)")
    p.add_argument("--trace-summarize", nargs=2, metavar=("TRACE_DIR", "OUT"),
                   help="per-launch-shape durations from a rocprofv3 --kernel-trace run of bench.py")
    p.add_argument("--trace-command", default="rocprofv3 --kernel-trace --stats -d OUT -o run --output-format csv "
                   "-- python3 REPO/bench.py --steps 208 --warmup 26 --no-cpu-baseline --no-stream --no-verify "
                   "--no-down",
                   help="the profiling command, recorded in the trace summary")
    return p.parse_args()


def kernel_source_hash() -> str:
    """sha256 over the HIP sources and headers the kernels are built from."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "quantized_decode_q4g128_amd")
    for path in sorted(glob.glob(os.path.join(pkg, "csrc", "*")) + [os.path.join(pkg, "build.py")]):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class RawCalls:
    """Launches through the C ABI with prepared pointers (no per-call Python
    checks), so that streams of many launches are not limited by the host."""

    def __init__(self, torch, q):
        self.torch, self.q, self.L = torch, q, q.lib()
        self.keep = []

    def prepare(self, case, copies, splits=None):
        """Device copies of the case's weights; returns a list of launch closures,
        one per copy."""
        torch, q, L = self.torch, self.q, self.L
        dev = torch.device("cuda:0")
        wt = case.weights
        W = torch.from_numpy(wt.W.view(np.int32)).to(dev)
        s = torch.from_numpy(wt.scale.view(np.int16)).to(dev)
        m = torch.from_numpy(wt.mn.view(np.int16)).to(dev)
        x = torch.from_numpy(case.x.view(np.int16)).to(dev)
        y = torch.empty((case.M, case.N), dtype=torch.float32, device=dev)
        if splits is None:
            splits = q.q4g128_splitk_default_splits(case.K, case.N)
        ws_bytes = q.q4g128_splitk_workspace_bytes(case.M, case.N, splits) if splits > 1 else 0
        ws = torch.empty(max(ws_bytes, 4) // 4, dtype=torch.float32, device=dev)
        sets = [(W, s, m)] + [(W.clone(), s.clone(), m.clone()) for _ in range(copies - 1)]
        self.keep += [x, y, ws, sets]
        self.ys = getattr(self, "ys", [])
        M, K, N = case.M, case.K, case.N
        calls = []
        for Wi, si, mi in sets:
            if splits > 1:
                args = (x.data_ptr(), M, K, Wi.data_ptr(), si.data_ptr(), mi.data_ptr(), N, y.data_ptr(),
                        splits, ws.data_ptr(), ws_bytes)
                calls.append(lambda st, a=args: L.q4g128_gemm_splitk(*a, st))
            else:
                args = (x.data_ptr(), M, K, Wi.data_ptr(), si.data_ptr(), mi.data_ptr(), N, y.data_ptr())
                calls.append(lambda st, a=args: L.q4g128_gemm(*a, st))
        self.ys.append((calls, y))
        self.sets_of = getattr(self, "sets_of", [])
        self.sets_of.append((calls, sets, case.K, case.N))
        return calls, splits

    def rows_on(self, calls, x_bits):
        """Launch closures for the product of other rows x (bf16 bits [M][K])
        on the weight copies of an existing launch list (q4g128_gemm, K not
        split): only x and M differ."""
        torch, L = self.torch, self.L
        dev = torch.device("cuda:0")
        sets, K, N = next((st, k, n) for c, st, k, n in self.sets_of if c is calls)
        M = x_bits.shape[0]
        x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        self.keep += [x, y]
        return [lambda st, a=(x.data_ptr(), M, K, Wi.data_ptr(), si.data_ptr(), mi.data_ptr(), N, y.data_ptr()):
                L.q4g128_gemm(*a, st) for Wi, si, mi in sets]

    def y_of(self, calls):
        """The output tensor the launch list writes."""
        return next(y for c, y in self.ys if c is calls)


def warm_up(torch, seq, seconds=WARM_S):
    """Passes over `seq` for about `seconds`: the first passes over freshly
    allocated weight copies run slower than the steady state, and an idle GPU
    starts at low clocks."""
    st = torch.cuda.current_stream().cuda_stream
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for c in seq:
            if c(st) != 0:
                raise RuntimeError("launch failed")
        torch.cuda.synchronize()


def timed_calls(torch, seq, reps, warmup, warm_s=WARM_S):
    """Milliseconds for `reps` passes over the launch sequence `seq`, bracketed
    by HIP events on the launching stream, after `warm_s` seconds and
    `warmup` passes of untimed launches."""
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    if warm_s > 0:
        warm_up(torch, seq, warm_s)
    for _ in range(warmup):
        for c in seq:
            if c(st) != 0:
                raise RuntimeError("launch failed")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(reps):
        for c in seq:
            c(st)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def timed_launches(torch, seq, n, warmup, warm_s=WARM_S):
    """Milliseconds for exactly `n` launches, launch i on copy i % len(seq)
    (cycling through the weight copies, no rounding to whole passes),
    bracketed by HIP events on the launching stream, after `warm_s` seconds
    and `warmup` untimed launches."""
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    if warm_s > 0:
        warm_up(torch, seq, warm_s)
    for i in range(warmup):
        if seq[i % len(seq)](st) != 0:
            raise RuntimeError("launch failed")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(n):
        seq[i % len(seq)](st)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def per_call_distribution(torch, seq, n):
    """Per-launch time distribution over at least `n` launches: batches of
    one pass over the weight copies (len(seq) launches, back to back), an
    event between batches, so a batch's time divided by its launches is one
    sample (events between single launches cost ~3 us each here, more than
    the spread they would show).  Returns microseconds per launch: median,
    min, p90 and mean over the batches."""
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    warm_up(torch, seq, WARM_S)
    nb = max(1, -(-n // len(seq)))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for b in range(nb):
        for c in seq:
            c(st)
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    dt = np.array([ev[b].elapsed_time(ev[b + 1]) * 1e3 / len(seq) for b in range(nb)])
    return {"launches": nb * len(seq), "batches": nb, "launches_per_batch": len(seq),
            "median_us": round(float(np.median(dt)), 3), "min_us": round(float(dt.min()), 3),
            "p90_us": round(float(np.percentile(dt, 90)), 3), "mean_us": round(float(dt.mean()), 3)}


def trace_reading(kernel_prefix):
    """Median and mean duration of the dominant launch shape of a kernel in
    the committed rocprofv3 trace summary, when that summary was taken on the
    current kernel sources (else None)."""
    if not os.path.exists(TRACE_SUMMARY):
        return None
    src, best = None, None
    with open(TRACE_SUMMARY) as f:
        for line in f:
            if line.startswith("# kernel_source_hash:"):
                src = line.split(":", 1)[1].strip()
            if line.startswith("#") or "|" not in line:
                continue
            cols = [c.strip() for c in line.split("|")]
            if not cols[0].split("::")[-1].startswith(kernel_prefix):
                continue
            n = int(cols[3])
            if best is None or n > best[0]:
                best = (n, float(cols[4]), float(cols[5]), cols[0])
    if best is None or src != kernel_source_hash():
        return None
    return {"kernel": best[3], "launches": best[0], "mean_us": best[1], "median_us": best[2],
            "file": os.path.relpath(TRACE_SUMMARY, ROOT)}


def measure_verify_ratios(torch, raw, dec_calls, ver_calls, ver_bytes, steps, warmup, passes=3):
    """Verify steps against the decode step on the gate/up shape: M = 7 (the
    verify workload), M = 9 (a draft of 8 tokens plus the next) and M = 16
    (the MFMA tile's rows), and the rest of the sweep M = 2..8 (on the decode
    step's weight copies), each `steps` launches on rotating weight copies,
    timed in `passes` interleaved passes together with M = 1; each ratio is
    of medians taken in the same passes, so box-to-box and drift effects
    cancel."""
    sets = {1: (dec_calls, None)}
    if ver_calls:
        sets[7] = (ver_calls, ver_bytes)
    for M in (9, 16):
        case = synth.make_random(M, 5120, 34816, 80 + M)
        B = synth.algorithmic_bytes(M, case.K, case.N)
        sets[M] = (raw.prepare(case, max(2, math.ceil(ROTATE_BYTES / B)), splits=1)[0], B)
    rows = synth.make_random(8, 5120, 1, 90).x
    for M in (2, 3, 4, 5, 6, 8):
        sets[M] = (raw.rows_on(dec_calls, rows[:M]), synth.algorithmic_bytes(M, 5120, 34816))
    t = {M: [] for M in sets}
    for _ in range(passes):
        for M, (calls, _) in sets.items():
            n = max(steps, len(calls))
            t[M].append(timed_launches(torch, calls, n, warmup) * 1e-3 / n)
    med = {M: sorted(v)[len(v) // 2] for M, v in t.items()}
    out = {}
    for M, (_, B) in sets.items():
        if M == 1:
            continue
        out[M] = {"us_per_call": round(med[M] * 1e6, 3), "GBps": round(B / med[M] / 1e9, 1), "bytes_per_call": B,
                  "time_ratio_vs_M1": round(med[M] / med[1], 4), "M1_us_same_passes": round(med[1] * 1e6, 3),
                  "passes": passes}
    return out


def measure_tiny(torch, q, steps, warmup):
    """The tiny workload (M=1, K=1024, N=1024; 563,200 bytes per call): a
    launch-bound product.  64 weight copies rotate (36 MB, so they sit in the
    last-level cache, as a product this small would)."""
    case = synth.make_case("tiny")
    B = synth.algorithmic_bytes(case.M, case.K, case.N)
    rc = RawCalls(torch, q)
    calls, splits = rc.prepare(case, 64)
    n = max(steps, len(calls))
    t = timed_launches(torch, calls, n, warmup) * 1e-3 / n
    return {"us_per_call": round(t * 1e6, 3), "GBps": round(B / t / 1e9, 1), "splits": splits,
            "bytes_per_call": B, "note": "launch-bound; weight copies resident in the last-level cache"}


def measure_down(torch, q, steps, warmup):
    """Decode down projection (M=1, K=17408, N=5120; split-K with the default
    split count, partial sums reduced in split order)."""
    case = synth.make_case("down")
    B = synth.algorithmic_bytes(case.M, case.K, case.N)
    rc = RawCalls(torch, q)
    calls, splits = rc.prepare(case, max(2, math.ceil(ROTATE_BYTES / B)))
    n = max(steps, len(calls))
    t = timed_launches(torch, calls, n, warmup) * 1e-3 / n
    # With the default split count equal to the one-launch form's K parts, a
    # one-row call is that single launch; other split counts add the reduce.
    one = splits == 1 or splits == q.q4g128_gemm_parts(case.K, case.N)
    return {"us_per_call": round(t * 1e6, 3), "GBps": round(B / t / 1e9, 1), "splits": splits,
            "bytes_per_call": B, "kernels_per_call": 1 if one else 2}


def measure_stream(torch, q, reps=5, warmup=2):
    """The full synthetic decode-step weight stream at M=1: 64 layers of four
    projections (5120->12288, 6144->5120, 5120->34816, 17408->5120), then the
    5120->131072 output projection, 257 launches back to back on one stream,
    every layer reading its own copy of the weights."""
    rc = RawCalls(torch, q)
    per_shape = []
    B_layer = 0
    for K, N, seed in synth.stream_shapes()[:-1]:
        case = synth.make_random(1, K, N, seed)
        calls, _ = rc.prepare(case, synth.STREAM_LAYERS)
        per_shape.append(calls)
        B_layer += synth.algorithmic_bytes(1, K, N)
    K, N, seed = synth.stream_shapes()[-1]
    head, _ = rc.prepare(synth.make_random(1, K, N, seed), 1)
    seq = [per_shape[j][layer] for layer in range(synth.STREAM_LAYERS) for j in range(len(per_shape))] + head
    B = synth.STREAM_LAYERS * B_layer + synth.algorithmic_bytes(1, K, N)
    ms = timed_calls(torch, seq, reps, warmup)
    t = ms * 1e-3 / reps
    out = {"launches_per_step": len(seq), "bytes_per_step": B, "ms_per_step": round(t * 1e3, 4),
           "GBps_wall": round(B / t / 1e9, 1), "steps_per_s": round(1.0 / t, 2),
           "note": "wall time of back-to-back launches, gaps between kernels included"}
    out["graph"] = graph_stream(torch, rc, seq, B, reps)
    del rc
    torch.cuda.empty_cache()
    return out


def dev_copies(torch, case, copies):
    """Device copies of a case's weights: [(W, scale, min)] * copies."""
    dev = torch.device("cuda:0")
    wt = case.weights
    W = torch.from_numpy(wt.W.view(np.int32)).to(dev)
    s = torch.from_numpy(wt.scale.view(np.int16)).to(dev)
    m = torch.from_numpy(wt.mn.view(np.int16)).to(dev)
    return [(W, s, m)] + [(W.clone(), s.clone(), m.clone()) for _ in range(copies - 1)]


def measure_epilogues(torch, q, steps, warmup):
    """The fused epilogues on their decode shapes, each call on its own weight
    copy: gate/up (M=1, K=5120, N=34816) with SwiGLU written as bf16, and down
    (M=1, K=17408, N=5120, default split count) with the split-K partials
    summed in the residual-add + RMSNorm."""
    L = q.lib()
    dev = torch.device("cuda:0")
    out = {}
    gu = synth.make_case("gateup")
    B = synth.algorithmic_bytes(gu.M, gu.K, gu.N)
    sets = dev_copies(torch, gu, max(2, math.ceil(ROTATE_BYTES / B)))
    x = torch.from_numpy(gu.x.view(np.int16)).to(dev)
    act = torch.empty((gu.M, gu.N // 2), dtype=torch.int16, device=dev)
    wsb = q.q4g128_swiglu_workspace_bytes(gu.M, gu.K, gu.N)
    ws = torch.empty(max(wsb, 4) // 4, dtype=torch.float32, device=dev)
    calls = [lambda st, a=(x.data_ptr(), gu.M, gu.K, W.data_ptr(), sc.data_ptr(), mn.data_ptr(), gu.N,
                           act.data_ptr(), ws.data_ptr(), wsb): L.q4g128_gemm_swiglu(*a, st) for W, sc, mn in sets]
    reps = max(1, steps // len(calls))
    t = timed_calls(torch, calls, reps, 1) * 1e-3 / (reps * len(calls))
    Bo = B - 4 * gu.M * gu.N + 2 * gu.M * (gu.N // 2)           # y not written; bf16 act instead
    out["gateup_swiglu_M1"] = {"us_per_call": round(t * 1e6, 3), "GBps": round(Bo / t / 1e9, 1),
                               "bytes_per_call": Bo, "launches_per_call": 1}
    del sets
    dn = synth.make_case("down")
    B = synth.algorithmic_bytes(dn.M, dn.K, dn.N)
    sets = dev_copies(torch, dn, max(2, math.ceil(ROTATE_BYTES / B)))
    x = torch.from_numpy(dn.x.view(np.int16)).to(dev)
    rng = np.random.default_rng(63)
    r = torch.from_numpy((rng.standard_normal((dn.M, dn.N)) * 0.5).astype(np.float32)).to(dev)
    gamma = torch.from_numpy(synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(dn.N)).view(np.int16)).to(dev)
    h = torch.empty((dn.M, dn.N), dtype=torch.float32, device=dev)
    xo = torch.empty((dn.M, dn.N), dtype=torch.int16, device=dev)
    S = q.q4g128_splitk_default_splits(dn.K, dn.N)
    ws = q.q4g128_rmsnorm_workspace(dn.M, dn.N, S, dev)
    wsb = ws.numel() * 4
    one_launch = 1 < S == q.q4g128_gemm_parts(dn.K, dn.N) and dn.M == 1      # the one-launch form's condition
    calls = [lambda st, a=(x.data_ptr(), dn.M, dn.K, W.data_ptr(), sc.data_ptr(), mn.data_ptr(), dn.N, r.data_ptr(),
                           gamma.data_ptr(), 1e-6, h.data_ptr(), xo.data_ptr(), S, ws.data_ptr(), wsb):
             L.q4g128_gemm_rmsnorm(*a, st) for W, sc, mn in sets]
    reps = max(1, steps // len(calls))
    t = timed_calls(torch, calls, reps, 1) * 1e-3 / (reps * len(calls))
    Bo = B + 4 * dn.M * dn.N + 2 * dn.N + 2 * dn.M * dn.N       # + residual in, gamma, bf16 x_out
    out["down_rmsnorm_M1"] = {"us_per_call": round(t * 1e6, 3), "GBps": round(Bo / t / 1e9, 1),
                              "bytes_per_call": Bo, "splits": S, "launches_per_call": 1 if one_launch else 2}
    # The residual add alone (x_out NULL): the norm is left to the next product.
    calls = [lambda st, a=(x.data_ptr(), dn.M, dn.K, W.data_ptr(), sc.data_ptr(), mn.data_ptr(), dn.N, r.data_ptr(),
                           None, 1e-6, h.data_ptr(), None, S, ws.data_ptr(), wsb):
             L.q4g128_gemm_rmsnorm(*a, st) for W, sc, mn in sets]
    t = timed_calls(torch, calls, reps, 1) * 1e-3 / (reps * len(calls))
    Bo = B + 4 * dn.M * dn.N                                    # + residual in
    out["down_residual_M1"] = {"us_per_call": round(t * 1e6, 3), "GBps": round(Bo / t / 1e9, 1),
                               "bytes_per_call": Bo, "splits": S, "launches_per_call": 1 if one_launch else 2}
    del sets
    torch.cuda.empty_cache()
    # The norm inside the consuming product: q/k/v and gate/up + SwiGLU made
    # from fp32 h, against the same products on a ready bf16 x.
    hrow = torch.from_numpy((rng.standard_normal((1, 5120)) * 0.5).astype(np.float32)).to(dev)
    g5 = torch.from_numpy(synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(5120)).view(np.int16)).to(dev)
    x5 = torch.from_numpy(synth.to_bf16_bits(rng.standard_normal((1, 5120))).view(np.int16)).to(dev)
    for name, (K, N), sw in (("qkv", (5120, 12288), False), ("gateup_swiglu", (5120, 34816), True)):
        case = synth.make_random(1, K, N, 70 + N % 13)
        B = synth.algorithmic_bytes(1, K, N)
        sets = dev_copies(torch, case, max(2, math.ceil(ROTATE_BYTES / B)))
        o = torch.empty((1, N // 2), dtype=torch.int16, device=dev) if sw else \
            torch.empty((1, N), dtype=torch.float32, device=dev)
        wpb = q.q4g128_prenorm_workspace_bytes(1, K, N, sw)
        wsp = torch.empty(max(wpb, q.q4g128_swiglu_workspace_bytes(1, K, N) if sw else 0, 256) // 4,
                          dtype=torch.float32, device=dev)
        wpb = wsp.numel() * 4
        if sw:
            plain = [lambda st, a=(x5.data_ptr(), 1, K, W.data_ptr(), sc.data_ptr(), mn.data_ptr(), N, o.data_ptr(),
                                   wsp.data_ptr(), wpb): L.q4g128_gemm_swiglu(*a, st) for W, sc, mn in sets]
            pre = [lambda st, a=(hrow.data_ptr(), g5.data_ptr(), 1e-6, 1, K, W.data_ptr(), sc.data_ptr(),
                                 mn.data_ptr(), N, o.data_ptr(), wsp.data_ptr(), wpb):
                   L.q4g128_gemm_swiglu_prenorm(*a, st) for W, sc, mn in sets]
        else:
            plain = [lambda st, a=(x5.data_ptr(), 1, K, W.data_ptr(), sc.data_ptr(), mn.data_ptr(), N, o.data_ptr()):
                     L.q4g128_gemm(*a, st) for W, sc, mn in sets]
            pre = [lambda st, a=(hrow.data_ptr(), g5.data_ptr(), 1e-6, 1, K, W.data_ptr(), sc.data_ptr(),
                                 mn.data_ptr(), N, o.data_ptr(), wsp.data_ptr(), wpb):
                   L.q4g128_gemm_prenorm(*a, st) for W, sc, mn in sets]
        reps = max(1, steps // len(plain))
        res = {}
        for _ in range(2):                                      # interleaved, best of two
            for key, calls in (("plain", plain), ("prenorm", pre)):
                t = timed_calls(torch, calls, reps, 1) * 1e-3 / (reps * len(calls))
                res[key] = min(res.get(key, t), t)
        out[name + "_prenorm_M1"] = {"us_per_call": round(res["prenorm"] * 1e6, 3),
                                     "us_per_call_on_ready_x": round(res["plain"] * 1e6, 3),
                                     "extra_us": round((res["prenorm"] - res["plain"]) * 1e6, 3),
                                     "launches_per_call": 1}
        del sets, plain, pre
        torch.cuda.empty_cache()
    return out


def measure_chain(torch, q, reps=5, prenorm=True):
    """A decode step whose products feed each other as in a transformer layer
    (attention itself out of scope), with h the fp32 residual stream.
    prenorm (each norm made inside the product that consumes it):
        qkv   = RMSNorm(h) . W_qkv                 (5120 -> 12288)
        h    += a . W_o                             (6144 -> 5120, a a fixed
                                                     stand-in for the attention output)
        act   = silu(gate) * up of RMSNorm(h) . W_gu   (5120 -> 2 x 17408)
        h    += act . W_down                        (17408 -> 5120)
      then logits = RMSNorm(h) . W_head.
    postnorm (the norm after the product, split-K partials summed in it):
        qkv   = x . W_qkv
        h    += a . W_o;  x' = RMSNorm(h)
        act   = silu(gate) * up of x' . W_gu
        h    += act . W_down;  x = RMSNorm(h)
      then logits = x . W_head.
    64 layers, every layer on its own weight copies, then the 5120 -> 131072
    output projection.  Timed eager and as one replayed HIP graph; each replay
    starts from the same residual and must reproduce the eager outputs bit for
    bit."""
    L = q.lib()
    dev = torch.device("cuda:0")
    shapes = synth.stream_shapes()
    cases = [synth.make_random(1, K, N, seed) for K, N, seed in shapes]
    layers = synth.STREAM_LAYERS
    w = [dev_copies(torch, cases[j], layers) for j in range(4)]
    head = dev_copies(torch, cases[4], 1)[0]
    rng = np.random.default_rng(64)
    d = 5120
    h0 = torch.from_numpy((rng.standard_normal((1, d)) * 0.5).astype(np.float32)).to(dev)
    h = h0.clone()
    x = torch.from_numpy(synth.to_bf16_bits(rng.standard_normal((1, d))).view(np.int16)).to(dev)
    x0 = x.clone()
    a = torch.from_numpy(synth.to_bf16_bits(rng.standard_normal((1, 6144))).view(np.int16)).to(dev)
    xm = torch.empty((1, d), dtype=torch.int16, device=dev)
    act = torch.empty((1, 17408), dtype=torch.int16, device=dev)
    qkv = torch.empty((1, 12288), dtype=torch.float32, device=dev)
    logits = torch.empty((1, 131072), dtype=torch.float32, device=dev)
    g_o = torch.from_numpy(synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(d)).view(np.int16)).to(dev)
    g_d = torch.from_numpy(synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(d)).view(np.int16)).to(dev)
    g_h = torch.from_numpy(synth.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(d)).view(np.int16)).to(dev)
    S_o = q.q4g128_splitk_default_splits(6144, d)
    S_d = q.q4g128_splitk_default_splits(17408, d)
    wsn = q.q4g128_rmsnorm_workspace(1, d, max(S_o, S_d), dev)       # control block zero: the norms' own
    wsnb = wsn.numel() * 4
    wsb = max(q.q4g128_splitk_workspace_bytes(1, d, S_o), q.q4g128_splitk_workspace_bytes(1, d, S_d),
              q.q4g128_swiglu_workspace_bytes(1, 5120, 34816),
              q.q4g128_prenorm_workspace_bytes(1, 5120, 12288), q.q4g128_prenorm_workspace_bytes(1, 5120, 34816, True),
              q.q4g128_prenorm_workspace_bytes(1, 5120, 131072))
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    hp, gp = h.data_ptr(), None
    seq = []
    for l in range(layers):
        Wq, sq, mq = w[0][l]
        Wo, so, mo = w[1][l]
        Wg, sg, mg = w[2][l]
        Wd, sd, md = w[3][l]
        if prenorm:
            seq.append(lambda st, A=(hp, g_d.data_ptr(), 1e-6, 1, 5120, Wq.data_ptr(), sq.data_ptr(), mq.data_ptr(),
                                     12288, qkv.data_ptr(), ws.data_ptr(), wsb): L.q4g128_gemm_prenorm(*A, st))
            seq.append(lambda st, A=(a.data_ptr(), 1, 6144, Wo.data_ptr(), so.data_ptr(), mo.data_ptr(), d, hp, gp,
                                     1e-6, hp, None, S_o, wsn.data_ptr(), wsnb): L.q4g128_gemm_rmsnorm(*A, st))
            seq.append(lambda st, A=(hp, g_o.data_ptr(), 1e-6, 1, 5120, Wg.data_ptr(), sg.data_ptr(), mg.data_ptr(),
                                     34816, act.data_ptr(), ws.data_ptr(), wsb): L.q4g128_gemm_swiglu_prenorm(*A, st))
            seq.append(lambda st, A=(act.data_ptr(), 1, 17408, Wd.data_ptr(), sd.data_ptr(), md.data_ptr(), d, hp,
                                     gp, 1e-6, hp, None, S_d, wsn.data_ptr(), wsnb): L.q4g128_gemm_rmsnorm(*A, st))
            continue
        seq.append(lambda st, A=(x.data_ptr(), 1, 5120, Wq.data_ptr(), sq.data_ptr(), mq.data_ptr(), 12288,
                                 qkv.data_ptr()): L.q4g128_gemm(*A, st))
        seq.append(lambda st, A=(a.data_ptr(), 1, 6144, Wo.data_ptr(), so.data_ptr(), mo.data_ptr(), d, h.data_ptr(),
                                 g_o.data_ptr(), 1e-6, h.data_ptr(), xm.data_ptr(), S_o, wsn.data_ptr(), wsnb):
                   L.q4g128_gemm_rmsnorm(*A, st))
        seq.append(lambda st, A=(xm.data_ptr(), 1, 5120, Wg.data_ptr(), sg.data_ptr(), mg.data_ptr(), 34816,
                                 act.data_ptr(), ws.data_ptr(), wsb): L.q4g128_gemm_swiglu(*A, st))
        seq.append(lambda st, A=(act.data_ptr(), 1, 17408, Wd.data_ptr(), sd.data_ptr(), md.data_ptr(), d,
                                 h.data_ptr(), g_d.data_ptr(), 1e-6, h.data_ptr(), x.data_ptr(), S_d, wsn.data_ptr(),
                                 wsnb): L.q4g128_gemm_rmsnorm(*A, st))
    Wh, sh, mh = head
    if prenorm:
        seq.append(lambda st, A=(hp, g_h.data_ptr(), 1e-6, 1, 5120, Wh.data_ptr(), sh.data_ptr(), mh.data_ptr(),
                                 131072, logits.data_ptr(), ws.data_ptr(), wsb): L.q4g128_gemm_prenorm(*A, st))
    else:
        seq.append(lambda st, A=(x.data_ptr(), 1, 5120, Wh.data_ptr(), sh.data_ptr(), mh.data_ptr(), 131072,
                                 logits.data_ptr()): L.q4g128_gemm(*A, st))
    B = layers * sum(synth.algorithmic_bytes(1, K, N) for K, N, _ in shapes[:4]) + \
        synth.algorithmic_bytes(1, *shapes[4][:2])
    stream = torch.cuda.current_stream()

    def reset():
        h.copy_(h0)
        x.copy_(x0)

    def run_eager():
        st = torch.cuda.current_stream().cuda_stream      # the capture stream inside torch.cuda.graph
        for c in seq:
            if c(st) != 0:
                raise RuntimeError("chain launch failed: " + q.q4g128_last_error())

    reset()
    run_eager()
    torch.cuda.synchronize()
    ref = (logits.clone(), h.clone())
    finite = bool(torch.isfinite(logits).all() and torch.isfinite(h).all())
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    ms = 0.0
    for _ in range(reps):
        reset()
        torch.cuda.synchronize()
        t0.record(stream)
        run_eager()
        t1.record(stream)
        torch.cuda.synchronize()
        ms += t0.elapsed_time(t1)
    t_eager = ms * 1e-3 / reps
    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g):
        run_eager()
    same = True
    ms = 0.0
    for _ in range(reps):
        reset()
        logits.fill_(float("nan"))
        torch.cuda.synchronize()
        t0.record(stream)
        g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms += t0.elapsed_time(t1)
        same = same and torch.equal(logits, ref[0]) and torch.equal(h, ref[1])
    t_graph = ms * 1e-3 / reps
    # Kernels per call: the fused forms are one launch on these shapes at
    # M = 1 (splits = the one-launch form's K parts; the prenorm staging).
    one = S_o == q.q4g128_gemm_parts(6144, d) > 1 and S_d == q.q4g128_gemm_parts(17408, d) > 1
    out = {"calls_per_step": len(seq), "launches_per_step": len(seq) + (0 if one else 2 * layers),
           "norm": "prenorm (in the consuming product)" if prenorm else "postnorm (after the product)",
           "bytes_per_step": B,
           "ms_per_step": round(t_eager * 1e3, 4), "GBps_wall": round(B / t_eager / 1e9, 1),
           "graph": {"ms_per_step": round(t_graph * 1e3, 4), "GBps_wall": round(B / t_graph / 1e9, 1),
                     "replay_equals_eager": bool(same)},
           "outputs_finite": finite,
           "note": "products chained through the fused norms; weight bytes as the plain stream"}
    del w, head, g
    torch.cuda.empty_cache()
    return out


def graph_stream(torch, rc, seq, B, reps):
    """The same step captured once in a HIP graph and replayed; each replay's
    outputs must equal the eager run's bit for bit."""
    torch.cuda.synchronize()
    eager = [y.clone() for _, y in rc.ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream().cuda_stream
        for c in seq:
            c(st)
    stream = torch.cuda.current_stream()
    same = True
    for _ in range(2):                       # replays checked against the eager result
        for _, y in rc.ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        same = same and all(torch.equal(y, e) for (_, y), e in zip(rc.ys, eager))
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    t = t0.elapsed_time(t1) * 1e-3 / reps
    return {"ms_per_step": round(t * 1e3, 4), "GBps_wall": round(B / t / 1e9, 1),
            "replay_equals_eager": bool(same)}


QUANT_SHAPE = (34816, 5120)     # the gate/up matrix, [N][K] bf16 before quantization
QUANT_NCAND = 9                  # 9 x 9 clipped ranges per group
QUANT_SAMPLE_COLS = 64
QUANT_FLOPS_PER_TRY = 8          # per weight and candidate: sub, div, rint, mul, add, sub, mul, add


def measure_quantize(torch, q, reps=5, warmup=2):
    """The quantizer on the gate/up matrix: bf16 weights [34816][5120] drawn
    N(0, 0.02^2) with 0.1% of entries x25, into codes, scale and minimum with
    the 9 x 9 range search.  Returns the timing and, for the parity gate, the
    sampled columns' bf16 input and GPU outputs."""
    N, K = QUANT_SHAPE
    G = K // synth.GROUP
    w = synth.draw_dense_weights(synth.rng_for(61), N, K)
    dev = torch.device("cuda:0")
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    W = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    s = torch.empty((N, G), dtype=torch.int16, device=dev)
    m = torch.empty((N, G), dtype=torch.int16, device=dev)
    e = torch.empty((N, G), dtype=torch.float64, device=dev)
    L = q.lib()
    stream = torch.cuda.current_stream()
    args = (wd.data_ptr(), K, N, QUANT_NCAND, W.data_ptr(), s.data_ptr(), m.data_ptr(), e.data_ptr(),
            stream.cuda_stream)
    for _ in range(warmup):
        if L.q4g128_quantize(*args) != 0:
            raise RuntimeError("quantize launch failed: " + q.q4g128_last_error())
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(reps):
        L.q4g128_quantize(*args)
    t1.record(stream)
    torch.cuda.synchronize()
    t = t0.elapsed_time(t1) * 1e-3 / reps
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(62).choice(N, QUANT_SAMPLE_COLS - 2,
                                                                                   replace=False)]))
    ci = torch.from_numpy(cols).to(dev)
    gpu = tuple(a.index_select(0, ci).cpu().numpy() for a in (W, s, m, e))
    flops = N * G * QUANT_NCAND ** 2 * synth.GROUP * QUANT_FLOPS_PER_TRY
    info = {"workload": f"quantize the gate/up matrix, bf16 [N={N}][K={K}], {QUANT_NCAND}x{QUANT_NCAND} "
                        f"range search per 128-group",
            "ms_per_matrix": round(t * 1e3, 4), "groups_per_s": round(N * G / t, 1),
            "input_GBps": round(2 * N * K / t / 1e9, 2),
            "roofline": {"bound": "alu", "achieved": round(flops / t / 1e12, 3), "peak": PEAK_FP64_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(flops / t / 1e12 / PEAK_FP64_TFLOPS, 4),
                         "traffic": None, "kernel": "quantize_q4g128",
                         "flops_per_launch": flops,
                         "counting": "fp64, 8 per weight per candidate, a divide counted as one"}}
    del wd, W, s, m, e
    torch.cuda.empty_cache()
    return info, (np.ascontiguousarray(w[cols]), gpu)


PROBE_LINEAR_WAVES = 1024


def measure_read_ceiling(torch, case, reps=20):
    """What HBM delivers on this GPU to a pure read of the gate/up codes
    (K*N/2 bytes, no arithmetic): in the product's access pattern and work
    split (one 12-wave workgroup per CU owning an equal share of the rows,
    tiles of 16 rows, 128 contiguous bytes per row per step) and read contiguously
    (1 KB per wave per step, 1024 waves).  Each launch reads its own copy of
    the codes, as the timed product does."""
    import ctypes
    from quantized_decode_q4g128_amd.build import PROBE_PATH
    if not os.path.exists(PROBE_PATH):
        return None
    P = ctypes.CDLL(PROBE_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    P.q4g128_probe_sink_words.argtypes = [ci, ci, ci]
    P.q4g128_probe_sink_words.restype = ctypes.c_size_t
    P.q4g128_probe_tile_read.argtypes = [vp, ci, ci, vp, vp]
    P.q4g128_probe_linear_read.argtypes = [vp, ci, ci, ci, vp, vp]
    dev = torch.device("cuda:0")
    K, N = case.K, case.N
    B = K * N // 2
    W = torch.from_numpy(case.weights.W.view(np.int32)).to(dev)
    copies = [W] + [W.clone() for _ in range(max(2, math.ceil(ROTATE_BYTES / B)) - 1)]
    sink = torch.empty(P.q4g128_probe_sink_words(K, N, PROBE_LINEAR_WAVES), dtype=torch.int32, device=dev)
    tile = [lambda st, w=w: P.q4g128_probe_tile_read(w.data_ptr(), K, N, sink.data_ptr(), st) for w in copies]
    lin = [lambda st, w=w: P.q4g128_probe_linear_read(w.data_ptr(), K, N, PROBE_LINEAR_WAVES, sink.data_ptr(), st)
           for w in copies]
    out = {"bytes_per_launch": B}
    for name, calls in (("tile_pattern", tile), ("linear", lin)):
        passes = max(1, reps * 13 // len(calls))
        t = timed_calls(torch, calls, passes, 2) * 1e-3 / (passes * len(calls))
        out[name] = {"us_per_launch": round(t * 1e6, 3), "GBps": round(B / t / 1e9, 1)}
    out["note"] = ("pure reads of the gate/up codes: tile_pattern = the product's work split (12-wave "
                   "workgroup per CU, 16-row tiles, 128 B per row per step (two groups), 2 steps in flight); "
                   "linear = 1 KB per wave per step, 1024 waves, 8 in flight; both with the non-temporal hint")
    del copies
    torch.cuda.empty_cache()
    # The same contiguous read over 4x the bytes (K = 20480): how far the
    # 89 MB figures are from the streaming rate once start-up is amortised.
    K4 = 4 * K
    B4 = K4 * N // 2
    g = torch.Generator(device=dev)
    g.manual_seed(97)
    big = [torch.randint(-2**31, 2**31 - 1, (N, K4 // 8), dtype=torch.int32, device=dev, generator=g)
           for _ in range(max(2, math.ceil(ROTATE_BYTES / B4)))]
    lin4 = [lambda st, w=w: P.q4g128_probe_linear_read(w.data_ptr(), K4, N, PROBE_LINEAR_WAVES, sink.data_ptr(), st)
            for w in big]
    passes = max(1, reps * 13 // len(lin4))
    t = timed_calls(torch, lin4, passes, 2) * 1e-3 / (passes * len(lin4))
    out["linear_4x"] = {"bytes_per_launch": B4, "us_per_launch": round(t * 1e6, 3), "GBps": round(B4 / t / 1e9, 1)}
    del big, lin4
    torch.cuda.empty_cache()
    return out


def measure_product_vs_probe(torch, q, reps=20):
    """The product at M = 1, N = 34816 for K = 3072, 5120 and 7168 (the same
    tiles per CU, loop length proportional to K) beside the tile-pattern read
    probe on the same codes: `extra_us`, product minus probe, is what a
    launch of the product costs beyond reading its codes in the same
    pattern (its scales and minimums, x staging, arithmetic, tail).  Weights
    are seeded random codes with constant scales and minimums (the time
    does not depend on the values); each launch reads its own copy."""
    import ctypes
    from quantized_decode_q4g128_amd.build import PROBE_PATH
    if not os.path.exists(PROBE_PATH):
        return None
    P = ctypes.CDLL(PROBE_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    P.q4g128_probe_sink_words.argtypes = [ci, ci, ci]
    P.q4g128_probe_sink_words.restype = ctypes.c_size_t
    P.q4g128_probe_tile_read.argtypes = [vp, ci, ci, vp, vp]
    dev = torch.device("cuda:0")
    L = q.lib()
    N = 34816
    sink = torch.empty(P.q4g128_probe_sink_words(0, N, PROBE_LINEAR_WAVES), dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(98)
    out = {}
    for K in (3072, 5120, 7168):
        G = K // 128
        B = synth.algorithmic_bytes(1, K, N)
        x = torch.randint(-2**15, 2**15 - 1, (1, K), dtype=torch.int16, device=dev, generator=g) & 0x3FFF
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        sets = [(torch.randint(-2**31, 2**31 - 1, (N, K // 8), dtype=torch.int32, device=dev, generator=g),
                 torch.full((N, G), 0x3C24, dtype=torch.int16, device=dev),
                 torch.full((N, G), -0x425C, dtype=torch.int16, device=dev))
                for _ in range(max(2, math.ceil(ROTATE_BYTES / B)))]
        prod = [lambda st, a=(x.data_ptr(), 1, K, W.data_ptr(), s.data_ptr(), m.data_ptr(), N, y.data_ptr()):
                L.q4g128_gemm(*a, st) for W, s, m in sets]
        probe = [lambda st, w=W: P.q4g128_probe_tile_read(w.data_ptr(), K, N, sink.data_ptr(), st)
                 for W, _, _ in sets]
        passes = max(1, reps * 13 // len(sets))
        # First passes over fresh allocations run slow (~2 us per launch at
        # first): warm both over every copy, then alternate and keep the best.
        timed_calls(torch, prod, 1, 4)
        timed_calls(torch, probe, 1, 4)
        tp = tr = float("inf")
        for _ in range(2):
            tp = min(tp, timed_calls(torch, prod, passes, 1) * 1e-3 / (passes * len(sets)))
            tr = min(tr, timed_calls(torch, probe, passes, 1) * 1e-3 / (passes * len(sets)))
        out[str(K)] = {"product_us": round(tp * 1e6, 3), "product_GBps": round(B / tp / 1e9, 1),
                       "tile_probe_us": round(tr * 1e6, 3), "tile_probe_GBps": round(K * N // 2 / tr / 1e9, 1),
                       "extra_us": round((tp - tr) * 1e6, 3)}
        del sets, prod, probe
        torch.cuda.empty_cache()
    out["note"] = ("M=1, N=34816: the product (algorithmic bytes) and the tile-pattern read probe (codes only) "
                   "on the same seeded random codes; extra_us = product - probe")
    return out


def cpu_baseline(dec_case, budget_s, y_dec, ver_case=None, y_ver=None, quant=None):
    """The CPU leg, the only part of the benchmark that runs the fp64 oracle:
    it times the oracle on the decode workload (when budget_s > 0) and
    computes the references the parity gate compares the GPU results with
    (decode and verify products within tolerance; the quantizer's sampled
    columns bit for bit).  Returns (baseline or None, {check: pass?})."""
    import oracle
    orc = oracle.load()
    wt = dec_case.weights
    y, a = orc.gemm(dec_case.x, wt.W, wt.scale, wt.mn)
    checks = {"decode_M1": bool(oracle.within_tolerance(y_dec, y, a).all())}
    if y_ver is not None:
        yv, av = orc.gemm(ver_case.x, ver_case.weights.W, ver_case.weights.scale, ver_case.weights.mn)
        checks["verify_M7"] = bool(oracle.within_tolerance(y_ver, yv, av).all())
    if quant is not None:
        w_cols, gpu = quant
        ref = orc.quantize(w_cols, QUANT_NCAND)
        checks["quantize"] = all(np.array_equal(np.ascontiguousarray(g).view(np.uint8),
                                                np.ascontiguousarray(r).view(np.uint8)) for g, r in zip(gpu, ref))
    if budget_s <= 0:
        return None, checks
    t0 = time.perf_counter()
    orc.gemm(dec_case.x, wt.W, wt.scale, wt.mn)
    reps = 1
    while time.perf_counter() - t0 < budget_s and reps < 1000:
        orc.gemm(dec_case.x, wt.W, wt.scale, wt.mn)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    B = synth.algorithmic_bytes(dec_case.M, dec_case.K, dec_case.N)
    # One thread, on a column sample of the same input (a bounded time).
    cols = np.arange(0, dec_case.N, 16, dtype=np.int64)
    t1 = time.perf_counter()
    orc.gemm(dec_case.x, wt.W, wt.scale, wt.mn, cols=cols, nthreads=1)
    dt1 = (time.perf_counter() - t1) * dec_case.N / cols.size
    case = dec_case
    return {"value": round(B / dt / 1e9, 4), "unit": "GB/s", "cores": orc.max_threads(), "kind": "oracle",
            "sample": f"{reps} full fp64 oracle calls on the same M={case.M} K={case.K} N={case.N} "
                      f"input ({dt * 1e3:.1f} ms per call, {reps * dt:.1f} s in all)",
            "one_thread": {"value": round(B / dt1 / 1e9, 4), "unit": "GB/s",
                           "sample": f"every 16th column ({cols.size} of {case.N}) on 1 thread, scaled to all N"},
            "per_config": oracle_per_config(orc, ver_case)}, \
        checks


def oracle_per_config(orc, ver_case, min_s=0.3):
    """The oracle (all threads) on the other workloads: tiny, down, the
    7-row verify, and the decode-step stream extrapolated from one call per
    distinct shape (64 x the four layer shapes + the output projection)."""
    def per_call(case):
        wt = case.weights
        t0 = time.perf_counter()
        n = 0
        while True:
            orc.gemm(case.x, wt.W, wt.scale, wt.mn)
            n += 1
            if time.perf_counter() - t0 >= min_s:
                return (time.perf_counter() - t0) / n
    out = {}
    for name, case in (("tiny", synth.make_case("tiny")), ("down_M1", synth.make_case("down")),
                       ("verify_M7", ver_case)):
        if case is None:
            continue
        dt = per_call(case)
        out[name] = {"GBps": round(synth.algorithmic_bytes(case.M, case.K, case.N) / dt / 1e9, 4),
                     "ms_per_call": round(dt * 1e3, 3)}
    t_step, b_step = 0.0, 0
    shapes = synth.stream_shapes()
    for i, (K, N, seed) in enumerate(shapes):
        c = synth.make_random(1, K, N, seed)
        reps = 1 if i == len(shapes) - 1 else synth.STREAM_LAYERS
        t_step += per_call(c) * reps
        b_step += synth.algorithmic_bytes(1, K, N) * reps
        del c
    out["decode_step_stream"] = {"GBps": round(b_step / t_step / 1e9, 4), "ms_per_step": round(t_step * 1e3, 1),
                                 "note": "one call per distinct shape, extrapolated to the 257-product step"}
    return out


def env_info(torch):
    """The device, the software stack and the GPU clock state (rocm-smi's
    report, read after the GPU legs; None where unavailable)."""
    import shutil
    import subprocess
    props = torch.cuda.get_device_properties(0)
    info = {"device": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip": torch.version.hip, "torch": torch.__version__,
            "rocm": None, "clocks": None}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        pass
    exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    try:
        r = subprocess.run([exe, "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        card = next(iter(json.loads(r.stdout).values()))
        info["clocks"] = {k.strip().rstrip(":"): v for k, v in card.items()
                          if "clk" in k.lower() or "clock" in k.lower()}
    except Exception:
        pass
    return info


# ---- HBM traffic from counters ------------------------------------------------

def pmc_case(shape):
    """The counter workload's case: the decode gate/up projection, or seeded
    random weights of another (K, N) at M=1."""
    if shape is None or tuple(shape) == (5120, 34816):
        return synth.make_case("gateup")
    K, N = shape
    return synth.make_random(1, K, N, 700 + K // 128 + N % 997)


def pmc_workload(shape=None):
    """One elementwise copy of COPY_BYTES (the calibration: it reads and
    writes exactly that many bytes), then PMC_LAUNCHES launches of the
    product (M=1, default split count) over rotating weight copies."""
    import torch
    import quantized_decode_q4g128_amd as q
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1, out=dst)              # an elementwise kernel: reads and writes COPY_BYTES
    torch.cuda.synchronize()
    case = pmc_case(shape)
    raw = RawCalls(torch, q)
    calls, _ = raw.prepare(case, max(2, math.ceil(ROTATE_BYTES / synth.algorithmic_bytes(case.M, case.K, case.N))),
                           splits=None if shape else 1)
    st = torch.cuda.current_stream().cuda_stream
    for i in range(PMC_LAUNCHES):
        calls[i % len(calls)](st)
    torch.cuda.synchronize()
    print(f"pmc workload: copy {COPY_BYTES} B, {PMC_LAUNCHES} launches of {KERNEL}", flush=True)


def _counter_per_dispatch(d, name_filter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if name_filter(r["Kernel_Name"]):
                per[int(r["Dispatch_Id"])] = per.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def pmc_summarize(fetch_dir, write_dir, out, shape=None):
    is_kernel = lambda n: KERNEL in n and "streamk" not in n and "splitk" not in n
    is_copy = lambda n: "MulFunctor" in n
    lines = {}
    for label, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        k = _counter_per_dispatch(d, is_kernel)
        c = _counter_per_dispatch(d, is_copy)
        if not k or not c:
            raise SystemExit(f"{label}: missing dispatches (kernel {len(k)}, copy {len(c)})")
        copy_kib = max(c)                   # the calibration copy
        factor = (COPY_BYTES / 1024.0) / copy_kib
        steady = k[len(k) // 4:]            # skip the first launches
        lines[label] = (float(np.mean(steady)), copy_kib, factor, len(steady))
    case = pmc_case(shape)
    B = synth.algorithmic_bytes(case.M, case.K, case.N)
    sh = f" --pmc-shape {case.K} {case.N}" if shape else ""
    what = ("the decode gate/up projection (M=1 K=5120 N=34816)" if not shape else
            f"the product M=1 K={case.K} N={case.N} (default split count: one launch)")
    fetch_b = lines["FETCH_SIZE"][0] * 1024 * lines["FETCH_SIZE"][2]
    write_b = lines["WRITE_SIZE"][0] * 1024 * lines["WRITE_SIZE"][2]
    with open(out, "w") as f:
        f.write(f"# HBM traffic of {KERNEL} on {what}\n")
        f.write("# commands (from the repository root; rocprofv3 run from /tmp with TMPDIR=/tmp):\n")
        f.write("#   rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o run --output-format csv -- "
                f"python3 bench.py --pmc-workload{sh}\n")
        f.write("#   rocprofv3 --pmc WRITE_SIZE -d OUT/write -o run --output-format csv -- "
                f"python3 bench.py --pmc-workload{sh}\n")
        f.write(f"#   python3 bench.py --pmc-summarize OUT/fetch OUT/write {os.path.relpath(out, ROOT)}{sh}\n")
        f.write("# calibration: one device copy of copy_bytes; factor = copy_bytes / counter reading\n")
        f.write(f"kernel_source_hash: {kernel_source_hash()}\n")
        f.write(f"copy_bytes: {COPY_BYTES}\n")
        for label in ("FETCH_SIZE", "WRITE_SIZE"):
            mean, copy_kib, factor, n = lines[label]
            f.write(f"{label}_kernel_kib_per_dispatch: {mean:.1f}\n")
            f.write(f"{label}_kernel_dispatches_averaged: {n}\n")
            f.write(f"{label}_copy_kib: {copy_kib:.1f}\n")
            f.write(f"{label}_factor: {factor:.4f}\n")
        f.write(f"fetch_bytes_per_launch: {fetch_b:.0f}\n")
        f.write(f"write_bytes_per_launch: {write_b:.0f}\n")
        f.write(f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}\n")
        f.write(f"algorithmic_bytes_per_launch: {B}\n")
        f.write(f"traffic_over_algorithmic: {(fetch_b + write_b) / B:.4f}\n")
    print(open(out).read())


def trace_summarize(trace_dir, out, command):
    """Per-launch-shape kernel durations from a rocprofv3 --kernel-trace run
    (launches of one kernel with different LDS sizes or grids are listed
    apart: the M=1 and M=7 launches of the product differ in LDS)."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    rows = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            key = (name, int(r["LDS_Block_Size"]), int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]),
                   int(r["Workgroup_Size_X"]))
            rows.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    with open(out, "w") as f:
        f.write("# rocprofv3 kernel trace of bench.py on one MI355X (gfx950), per launch shape\n")
        f.write("# command (rocprofv3 started from /tmp with TMPDIR=/tmp; REPO = repository root):\n")
        f.write(f"#   {command}\n")
        f.write(f"#   python3 bench.py --trace-summarize OUT {os.path.relpath(out, ROOT)}\n")
        f.write(f"# kernel_source_hash: {kernel_source_hash()}\n")
        f.write("# kernel | grid x,y | workgroup | launches | avg us | median us | min us | p90 us | max us\n")
        for key in sorted(rows, key=lambda k: -sum(rows[k])):
            v = np.array(rows[key])
            f.write(f"{key[0]} | {key[2]},{key[3]} | {key[4]} | {len(v)} | {v.mean():.3f} | {np.median(v):.3f} | "
                    f"{v.min():.3f} | {np.percentile(v, 90):.3f} | {v.max():.3f}\n")
    print(open(out).read())


def traffic_from_summary():
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing or was taken on other kernel sources."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    kv = {}
    with open(PMC_SUMMARY) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


# ---- main --------------------------------------------------------------------

def main():
    args = parse()
    if args.pmc_summarize:
        pmc_summarize(*args.pmc_summarize, shape=args.pmc_shape)
        return
    if args.trace_summarize:
        trace_summarize(*args.trace_summarize, args.trace_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the product runs on one GPU's "
              f"share of the weights and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_decode_q4g128_amd as q
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.pmc_workload:
        pmc_workload(args.pmc_shape)
        return
    if args.stream_only:
        print(json.dumps({"decode_step_stream": measure_stream(torch, q)}))
        return

    dec_case = synth.make_case("gateup")
    ver_case = synth.make_case("verify", 7)
    B_dec = synth.algorithmic_bytes(dec_case.M, dec_case.K, dec_case.N)
    B_ver = synth.algorithmic_bytes(ver_case.M, ver_case.K, ver_case.N)
    # Launches through the C ABI with prepared pointers: per-call Python
    # checks would otherwise leave the GPU waiting on the host between
    # 20-microsecond kernels.
    raw = RawCalls(torch, q)
    dec_calls, _ = raw.prepare(dec_case, max(2, math.ceil(ROTATE_BYTES / B_dec)), splits=1)
    ver_calls = None if args.no_verify else raw.prepare(ver_case, max(2, math.ceil(ROTATE_BYTES / B_ver)),
                                                         splits=1)[0]

    # Parity gate on the exact launches that get timed (first rotation set).
    st = torch.cuda.current_stream().cuda_stream
    if dec_calls[0](st) != 0 or (ver_calls and ver_calls[0](st) != 0):
        raise SystemExit("launch failed: " + q.q4g128_last_error())
    torch.cuda.synchronize()
    y_dec = raw.y_of(dec_calls).cpu().numpy()
    y_ver = raw.y_of(ver_calls).cpu().numpy() if ver_calls else None

    # Bring the GPU out of its idle clocks (setting up the inputs kept it idle
    # for seconds) before anything is timed: ~0.5 s of decode launches.
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        for c in dec_calls:
            c(st)
        torch.cuda.synchronize()
    n_dec = args.steps                            # exactly the launches asked for, cycling the copies
    wall_d = timed_launches(torch, dec_calls, n_dec, args.warmup)
    ms_step = wall_d / n_dec
    t_dec = wall_d * 1e-3 / n_dec                 # s per launch (back to back)
    gbps = B_dec * n_dec / (wall_d * 1e-3) / 1e9
    achieved = B_dec / t_dec / 1e9
    dist = per_call_distribution(torch, dec_calls, max(DIST_CALLS, args.steps))
    verify, wider, sweep = None, None, None
    if ver_calls:
        vr = measure_verify_ratios(torch, raw, dec_calls, ver_calls, B_ver, args.steps, args.warmup)
        verify = vr.pop(7)
        wider = {f"M{M}": vr.pop(M) for M in (9, 16)}
        sweep = {f"M{M}": vr[M] for M in sorted(vr)}
    traffic = traffic_from_summary()
    ceiling = None if args.no_read_ceiling else measure_read_ceiling(torch, dec_case)
    if ceiling is not None:
        ceiling["product_vs_probe"] = measure_product_vs_probe(torch, q)
    down = None if args.no_down else measure_down(torch, q, args.steps, args.warmup)
    tiny = measure_tiny(torch, q, args.steps, args.warmup)
    stream_step = measure_stream(torch, q) if not args.no_stream else None
    epilogues = None if args.no_epilogues else measure_epilogues(torch, q, args.steps, args.warmup)
    chain = measure_chain(torch, q) if not (args.no_stream or args.no_epilogues) else None
    chain_post = measure_chain(torch, q, prenorm=False) if chain is not None else None
    quant, quant_out = (None, None) if args.no_quantize else measure_quantize(torch, q)
    env = env_info(torch)            # after every GPU leg: rocm-smi leaves the GPU idle for a second or two

    # The CPU leg last: oracle baseline and the parity references.
    cpu, checks = cpu_baseline(dec_case, 0.0 if args.no_cpu_baseline else args.cpu_seconds, y_dec,
                               ver_case, y_ver, quant_out)
    ok_dec, ok_ver = checks["decode_M1"], checks.get("verify_M7")
    if verify is not None:
        if not ok_ver:
            verify["GBps"] = None
        if not (ok_ver and ok_dec):
            verify["time_ratio_vs_M1"] = None
    if quant is not None:
        quant["parity"] = "pass" if checks["quantize"] else "FAIL"
        if not checks["quantize"]:
            quant["roofline"]["achieved"] = quant["roofline"]["frac"] = None

    line = {
        "metric": METRIC,
        "value": round(gbps, 1) if ok_dec else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n_dec,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode gate/up projection, int4-g128, M=1 K=5120 N=34816",
                   "M": 1, "K": 5120, "N": 34816, "bytes_per_step": B_dec,
                   "weight_copies_rotated": len(dec_calls), "accumulate": "fp32"},
        "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2) if ok_dec else None,
        "parity": {"decode_M1": "pass" if ok_dec else "FAIL",
                   "verify_M7": None if ok_ver is None else ("pass" if ok_ver else "FAIL")},
        "verify_M7": verify,
        "verify_wider": wider,
        "verify_sweep": sweep,
        "tiny_M1": tiny,
        "down_M1": down,
        "decode_step_stream": stream_step,
        "epilogues": epilogues,
        "decode_step_chain": chain,
        "decode_step_chain_postnorm": chain_post,
        "quantize": quant,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": round(traffic) if traffic is not None else None,
                     "kernel": KERNEL, "us_per_launch": round(t_dec * 1e6, 3),
                     "per_call": dist, "trace": trace_reading(KERNEL),
                     "algorithmic_bytes_per_launch": B_dec,
                     "frac_of_read_ceiling": (round(achieved / ceiling["tile_pattern"]["GBps"], 4)
                                              if ceiling else None)},
        "read_ceiling": ceiling,
        "cpu_baseline": cpu,
        "env": env,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

"""bench.py's host logic, no GPU needed: the refusal of more than one GPU,
and the arithmetic of the committed counter summary the bench reads its
HBM traffic from (each counter scaled by what it reads for a plain copy of
known size)."""
import glob
import os
import re
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""                   # no bench line


def summary(path):
    kv = {}
    with open(path) as f:
        head = f.readline()
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    m = re.search(r"M=1 K=(\d+) N=(\d+)", head)
    return kv, int(m.group(1)), int(m.group(2))


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*_pmc.txt"))))
def test_counter_summary_arithmetic(path):
    kv, K, N = summary(path)
    copy_kib = {c: float(kv[f"{c}_copy_kib"]) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    factor = {c: float(kv[f"{c}_factor"]) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    per = {c: float(kv[f"{c}_kernel_kib_per_dispatch"]) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    copy_bytes = float(kv["copy_bytes"])
    for c in factor:                                   # factor = copy bytes / the counter's reading of the copy
        assert abs(factor[c] - copy_bytes / 1024.0 / copy_kib[c]) <= 1e-4 * factor[c]
    fetch, write = float(kv["fetch_bytes_per_launch"]), float(kv["write_bytes_per_launch"])
    assert abs(fetch - per["FETCH_SIZE"] * 1024 * factor["FETCH_SIZE"]) <= 1e-4 * fetch
    assert abs(write - per["WRITE_SIZE"] * 1024 * factor["WRITE_SIZE"]) <= 1e-4 * write + 1024
    alg = float(kv["algorithmic_bytes_per_launch"])
    assert alg == synth.algorithmic_bytes(1, K, N)
    traffic = float(kv["traffic_bytes_per_launch"])
    assert abs(traffic - (fetch + write)) <= 1.0
    assert abs(float(kv["traffic_over_algorithmic"]) - traffic / alg) <= 1e-4
    # what the kernel writes is y (fp32 [1][N]) and nothing else; what it
    # fetches is within 2% of its codes, scales, minimums and x (x once per
    # L2 weighs most on the smallest matrix)
    assert abs(write - 4 * N) <= 1024
    assert 1.0 <= fetch / (alg - 4 * N) <= 1.02

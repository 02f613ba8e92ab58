"""Build libq4g128.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Every HIP source is compiled with packed fp32 instructions disabled
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libq4g128.so")
PROBE_PATH = os.path.join(PKG, "libq4g128_probe.so")      # read-bandwidth probes, loaded by bench.py only
PROBE_SOURCE = os.path.join(CSRC, "q4g128_probe.hip")
SOURCES = [os.path.join(CSRC, "q4g128_kernels.hip"), os.path.join(CSRC, "q4g128_streamk.hip"),
           os.path.join(CSRC, "q4g128_quant.hip"), os.path.join(CSRC, "q4g128_api.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libq4g128.so)")


def compile_flags(arch: str = ARCH):
    return [f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE, "-I", CSRC]


def _scratch_users(msgs):
    """Kernels that the compiler's resource report shows using scratch."""
    users, name = [], None
    for line in msgs:
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            users.append((name, int(m.group(1))))
    return users


def build_library(out: str = LIB_PATH, extra_flags=(), quiet: bool = True) -> str:
    """Compile the library.  Fails if a kernel spills to scratch: a kernel
    with scratch gets fewer waves in flight and streams markedly slower."""
    tmp = out + ".tmp"
    cmd = ([hipcc()] + compile_flags() + list(extra_flags) + ["-Rpass-analysis=kernel-resource-usage", "-shared"]
           + SOURCES + ["-o", tmp])
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if l.strip() and noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    spills = _scratch_users(msgs)
    if spills:
        os.remove(tmp)
        raise RuntimeError("kernels use scratch (register spills): " + ", ".join(f"{n} {b} B/lane" for n, b in spills))
    if not quiet:
        print("\n".join(l for l in msgs if "remark" not in l))
    os.replace(tmp, out)
    return out


def build_probe(out: str = PROBE_PATH) -> str:
    """Compile the benchmark's read-bandwidth probes (a library of their own)."""
    tmp = out + ".tmp"
    cmd = [hipcc()] + compile_flags() + ["-shared", PROBE_SOURCE, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(quiet=False))
    print(build_probe())

"""Compile the C oracle (test infrastructure) with the host compiler.

``build_oracle()`` writes ``oracle/libq4g128_oracle.so``; ``plant=<n>`` builds a
copy with one deliberate mistake (see ``ORACLE_PLANT`` in the C source) for the
tests that show each pin catches a mistake.
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "q4g128_oracle.c")


def build_oracle(out: str | None = None, plant: int = 0, cc: str = "gcc") -> str:
    out = out or os.path.join(_HERE, "libq4g128_oracle.so")
    tmp = out + ".tmp"
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           f"-DORACLE_PLANT={int(plant)}", SOURCE, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle())

"""Builds the float64 CPU oracle library (TEST INFRASTRUCTURE ONLY).

Plain gcc with OpenMP; no fast-math, so every operation is IEEE double.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "recurrence.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")


def needs_build() -> bool:
    return (not os.path.exists(LIB_PATH)) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC)


def build_oracle(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_oracle(verbose=True))

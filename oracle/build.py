"""Build the CPU oracle (``liborc.so``) from ``orc.cpp`` with the host compiler.

    python -m oracle.build

Flags: -O2 without fast-math and -ffp-contract=off, so every binary32 and
binary64 operation of the oracle is one correctly rounded IEEE operation in
the order the source writes it (no fused multiply-adds); x86-64 does
floating point in SSE, so there is no extended-precision intermediate.
TEST INFRASTRUCTURE ONLY: built beside the HIP library, never linked with it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "orc.cpp")
LIB = os.path.join(HERE, "liborc.so")
FLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
         "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        raise RuntimeError("no host C++ compiler (g++) found: the oracle cannot be built")
    tmp = LIB + ".tmp"
    proc = subprocess.run([cxx, *FLAGS, SRC, "-o", tmp], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{proc.stdout}")
    if verbose and proc.stdout.strip():
        print(proc.stdout)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

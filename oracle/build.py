"""Build the C++ fp64 oracle (TEST INFRASTRUCTURE ONLY) with the host compiler.

Usage: ``python -m oracle.build`` (or ``build_oracle()``).  Produces
``oracle/liboracle.so`` from ``oracle/cpp_oracle.cpp`` with g++ and OpenMP.
The hot loops carry a Haswell (AVX2 + FMA) clone beside the baseline x86-64
one; the loader picks the clone the host supports.
"""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(verbose: bool = True) -> str:
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        raise RuntimeError("no host C++ compiler (g++) to build the oracle")
    tmp = LIB + ".tmp"
    cmd = [cxx, "-O3", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_oracle()

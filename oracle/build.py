"""Build of the C++ fp64 oracle (``liboracle.so``), host code only.

TEST INFRASTRUCTURE ONLY (see the package docstring).  g++ with OpenMP and
no floating-point contraction, so every product and sum is rounded on its
own, as the definitions are written.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

FLAGS = ["-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
         "-shared"]


def build(verbose: bool = False, out: str = LIB, plant: int = 0) -> str:
    """Compile the oracle; ``plant`` > 0 builds a copy with one planted
    mistake (for the tests that check that a pin catches it)."""
    tmp = out + ".tmp"
    cmd = ["g++", *FLAGS, *([f"-DORACLE_PLANT={plant}"] if plant else []), SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def ensure_built() -> str:
    """The oracle library, compiled first if it is missing or older than its source."""
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

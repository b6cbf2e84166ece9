"""Build the CPU oracle library (plain C, gcc).

TEST INFRASTRUCTURE ONLY: the oracle is used by the tests, the smoke check and
the benchmark's CPU-baseline leg; the product path never loads it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(HERE, "softmax_oracle.c"), os.path.join(HERE, "norm_oracle.c")]
LIBRARY = os.path.join(HERE, "libsoftmax_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle's C sources into libsoftmax_oracle.so; return its path.

    Strict IEEE double: no -ffast-math, no FMA contraction.
    """
    tmp = LIBRARY + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fPIC", "-shared", "-o", tmp, *SOURCES, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))

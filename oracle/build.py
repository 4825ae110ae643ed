"""Compile the C oracle into ``oracle/liboracle.so`` (host only, gcc + OpenMP).

Test infrastructure: the library is built beside its source so that the tests,
the smoke check and the CPU-baseline leg of the benchmark can load it.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "rawint4_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # x86-64-v3 (AVX2 + FMA) runs on every host that carries an MI355X; no
    # -ffast-math: the oracle relies on IEEE exp overflow behaviour.
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIBRARY + ".tmp", SOURCE, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))

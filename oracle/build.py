"""Build the CPU oracle (``liboracle.so``) with gcc.

Test infrastructure only: the oracle is compiled here so that tests,
``__graft_entry__.smoke()`` and the cpu_baseline leg of ``bench.py`` can load
it.  Building it is not using it.

Floating-point flags matter: the oracle's quantiser must take every FP32
rounding step the format recipe states, so contraction into FMA and any
fast-math reassociation are switched off.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "msa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

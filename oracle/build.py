"""Builds the CPU oracle library (test infrastructure only).

Plain gcc, -O2, OpenMP over independent outputs, no FMA contraction and no
fast-math, so that every binary32 operation in the quantisers is rounded on
its own exactly as the C source reads.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mmf_oracle.c")
LIB = os.path.join(HERE, "libmmf_oracle.so")

CMD = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
       "-fPIC", "-shared", SRC, "-o", LIB, "-lm"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = CMD[:-3] + ["-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

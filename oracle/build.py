"""Build the CPU oracle (plain C, gcc) into oracle/libmoe_oracle.so.

Test infrastructure only: the HIP library never links or loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

# -ffp-contract=off: no implicit fused multiply-adds; the oracle writes every
# fma it means as an explicit fmaf() call.
CMD = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
       "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB, SRC, "-lm"]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = CMD[:CMD.index("-o") + 1] + [tmp] + CMD[CMD.index("-o") + 2:]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

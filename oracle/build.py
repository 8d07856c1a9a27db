"""Compile the CPU oracle (plain C, gcc, OpenMP) into oracle/libw4moe_oracle.so.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use the
library this builds.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "w4moe_oracle.c")
LIB = os.path.join(HERE, "libw4moe_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

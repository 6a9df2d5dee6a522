"""Compile the fp64 C oracle into oracle/libkda_oracle.so (test infrastructure).

Built with gcc, -O2 and OpenMP, for the baseline x86-64 ISA so the same
library runs on any x86-64 host."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

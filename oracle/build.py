"""Build the C oracle (plain gcc, no GPU code) into oracle/liboracle.so.

Test infrastructure: compiling the checker is not using it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pagedkv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared",
        # keep the oracle's double arithmetic exactly as written: no
        # contraction of a*b+c into fma, no reassociation
        "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        SRC, "-o", LIB + ".tmp", "-lm", "-lpthread",
    ]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the C oracle (test infrastructure) into oracle/libzero_oracle.so.

Plain gcc, -O2 -ffp-contract=off, no -march and no fast-math, so every float
operation is a single IEEE binary32 operation with round-to-nearest-even.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libzero_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", os.path.join(HERE, "zero_oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the CPU oracle shared library (test infrastructure only).

gcc, -O2, no fast-math and no floating-point contraction, so each fp32
operation in dsi_oracle.c is one IEEE operation in the written order.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dsi_oracle.c")
LIB = os.path.join(HERE, "libdsi_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-Wno-unused-parameter", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

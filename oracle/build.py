"""Compile the CPU oracle (plain C) into ``oracle/liboracle.so``.

Test infrastructure: the oracle is loaded only by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  ``-ffp-contract=off`` forbids fused multiply-adds, so every
float expression rounds exactly as written; no fast-math flag is ever passed.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp8_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
        "-Wall", "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

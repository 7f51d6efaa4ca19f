"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle.so.

Test infrastructure: the oracle is built so the tests, the smoke check and the
benchmark's CPU-baseline leg can load it; nothing on the product path does.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ukv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

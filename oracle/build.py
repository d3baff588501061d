"""Compile the CPU oracle (``fp8w_oracle.c``) into ``liboracle.so`` with gcc.

Test infrastructure: the oracle is used by the test suite, the package smoke
check and the benchmark's CPU-baseline leg only.

IEEE semantics are required (the quantizer's fp32 division must be correctly
rounded), so no fast-math flags are used.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp8w_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

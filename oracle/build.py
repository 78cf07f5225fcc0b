"""Compile the CPU oracle (plain C) into oracle/libllmoe_oracle.so with gcc.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg load the result.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ll_moe_oracle.c")
LIB = os.path.join(HERE, "libllmoe_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

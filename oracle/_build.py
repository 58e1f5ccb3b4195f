"""Build the CPU oracle library (TEST INFRASTRUCTURE ONLY).

Compiles oracle/q4k_oracle.c with gcc into oracle/libq4k_oracle.so: plain
scalar C, -O2, no FMA contraction, no vectorisation flags beyond -O2.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4k_oracle.c")
LIB = os.path.join(HERE, "libq4k_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
        "-Wall", "-Wextra", "-shared", "-fPIC", SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

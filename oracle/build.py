"""Build the C++ oracle into ``oracle/libring_oracle.so`` (test infrastructure).

Compiled with plain g++ at -O2, strict IEEE arithmetic (no fast-math, no FMA
contraction) and no target-specific vector code, so that its binary64
arithmetic is exactly what the source says.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libring_oracle.so")
SRC = os.path.join(HERE, "ring_sim.cpp")


def build(verbose: bool = False) -> str:
    cmd = [
        "g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-fno-fast-math",
        "-ffp-contract=off", "-pthread", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

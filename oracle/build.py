"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so with g++.

The flags keep every fp32 product and sum individually rounded (-ffp-contract=off,
no fast-math) and target a portable x86-64 level so the library also runs on
hosts other than the one that built it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
           "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

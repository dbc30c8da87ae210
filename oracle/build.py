"""Compile the CPU oracle (oracle/blake3_oracle.c) into oracle/_b3oracle.so with gcc.

Test infrastructure only: the oracle verifies results and is never part of the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "blake3_oracle.c")
LIB = os.path.join(HERE, "_b3oracle.so")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Always recompiles; returns the path of the shared library."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread",
           *extra_flags, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

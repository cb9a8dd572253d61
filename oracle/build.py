"""Build the CPU oracle (test infrastructure) into oracle/libmoe_oracle.so.

Plain g++ with OpenMP; no HIP, no torch. Called by ``__graft_entry__.build()``
and, when the library is missing, by the oracle loader.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.cpp")
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

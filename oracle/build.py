"""Build the CPU oracle (TEST INFRASTRUCTURE) into oracle/libstrata_oracle.so.

Plain gcc, fp64, OpenMP over independent rows; no GPU code, no shared headers.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libstrata_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "strata_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

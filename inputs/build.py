"""Build the device side of the input generator into inputs/libstrata_inputs.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libstrata_inputs.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *HIP_FLAGS, "-o", tmp, os.path.join(HERE, "fill.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.DEVNULL)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

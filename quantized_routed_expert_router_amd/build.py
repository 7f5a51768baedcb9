"""Build the HIP library libstrata_moe.so (gfx950) in-tree.

hipcc compiles every csrc/*.hip translation unit for gfx950 and links one
shared library exporting the C ABI of include/strata_moe.h.
"""
import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libstrata_moe.so")
OBJ = os.path.join(HERE, "_build")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-fvisibility=hidden"]


def _quiet(stderr: str) -> str:
    keep = [ln for ln in stderr.splitlines() if "packed-fp32-ops" not in ln]
    return "\n".join(keep)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def cc(src):
        obj = os.path.join(OBJ, src[:-4] + ".o")
        cmd = ["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = _quiet(r.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg, flush=True)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(cc, srcs))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{_quiet(r.stderr)}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB, flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

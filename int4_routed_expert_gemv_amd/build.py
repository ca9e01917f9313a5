"""Builds libmoe.so (the HIP library behind include/moe.h) for gfx950, in-tree."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed FP32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    if p.returncode != 0:
        sys.stderr.write(text)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
    # hipcc's host pass does not know the packed-fp32 feature flag; drop that note
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds, in-tree for gfx950, libmoe.so (the HIP library behind include/moe.h
and include/moe_cache.h) and libmoe_probe.so (the measurement probes of
include/moe_probe.h, loaded by the benchmark only)."""
import glob
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
PROBE_DIR = os.path.join(HERE, "probe")
PROBE_LIB = os.path.join(HERE, "libmoe_probe.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed FP32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# per-source flags: the matrix-core kernels keep their MFMA results in
# ordinary vector registers, so the float32 scaling of each step's products
# reads them directly (no copies out of the accumulation registers)
EXTRA = {"expert_mfma.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def sources(folder=CSRC):
    return sorted(glob.glob(os.path.join(folder, "*.hip")))


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compiles every source (all at once, up to `jobs` in parallel), then
    links the product library and the probe library."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs = []
    libs = {LIB: [], PROBE_LIB: []}
    for lib, folder in ((LIB, CSRC), (PROBE_LIB, PROBE_DIR)):
        for src in sources(folder):
            obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
            libs[lib].append(obj)
            cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT)))
            if len(procs) >= jobs:
                _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    for lib, objs in libs.items():
        tmp = lib + ".tmp"
        subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs,
                               "-o", tmp])
        missing = kernels_without_code(tmp)
        if missing:
            os.remove(tmp)
            raise RuntimeError(f"{os.path.basename(lib)}: host code launches kernels that its "
                               f"gfx950 code object lacks: {missing}")
        os.replace(tmp, lib)
    return LIB


_STUB = re.compile(rb"_Z[A-Za-z0-9_]*__device_stub__[A-Za-z0-9_]*")
_PREFIX = "__device_stub__"


def _kernel_of_stub(sym: str):
    """The mangled kernel name of a host launch stub's: the stub's name with
    the prefix taken out of its identifier (lengths read in order, so the
    anonymous namespace's own digits are not mistaken for one)."""
    i = 3 if sym.startswith("_ZN") else 2
    while i < len(sym) and sym[i].isdigit():
        j = i
        while sym[j].isdigit():
            j += 1
        n = int(sym[i:j])
        ident = sym[j:j + n]
        if ident.startswith(_PREFIX):
            return sym[:i] + str(n - len(_PREFIX)) + ident[len(_PREFIX):] + sym[j + n:]
        i = j + n
    return None


def kernels_without_code(path: str) -> list:
    """Kernels whose host launch stub is in the library but whose kernel
    descriptor (name.kd) is not in its device code object. A library like
    that (e.g. host and device passes of one source that saw different
    versions of it) fails in the HIP runtime when it first loads the code
    object. Returns [] when the code object is not readable as plain text
    (no descriptor names at all)."""
    blob = open(path, "rb").read()
    kds = {k.decode() for k in re.findall(rb"([A-Za-z0-9_]+)\.kd", blob)}
    if not kds:
        return []
    missing = set()
    for m in _STUB.finditer(blob):
        name = _kernel_of_stub(m.group(0).decode())
        if name is not None and name not in kds:
            missing.add(name)
    return sorted(missing)


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

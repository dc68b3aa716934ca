"""Build libmoe_q4.so in-tree with hipcc for gfx950.

Flags:
  -O3 --offload-arch=gfx950          the only target
  -fhip-fp32-correctly-rounded-divide-sqrt, -fno-fast-math
                                     Q8_0 codes need IEEE division and rint
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                     no packed fp32 VALU instructions
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe_q4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
OBJDIR = os.path.join(PKG, "_build")
# the host pass does not know the GPU-only target feature; drop that one note
_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra=(), lib: str = LIB, objdir: str = OBJDIR, link_extra=()) -> str:
    """Compile every source (one hipcc per file, in parallel), then link the shared library."""
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *extra, *inc, "-c", src, "-o", obj])
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, *objs, "-o", lib + ".tmp"], verbose)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))

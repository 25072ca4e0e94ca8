"""Build the HIP library in-tree: sparse_expert_dispatch_amd/lib/libmoe_dispatch.so.

Every source under csrc/ is compiled for gfx950 with hipcc and linked into
one shared library exporting the C ABI of include/moe_dispatch.h.

    python -m sparse_expert_dispatch_amd.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libmoe_dispatch.so"
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.cpp", "router.hip", "select.hip", "route_map.hip", "permute.hip", "grouped_gemm.hip",
           "stats.hip", "backward.hip", "noalloc.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Every float operation is rounded on its own unless the source asks for
    # fmaf explicitly: the score transform must be reproducible bit for bit.
    "-ffp-contract=off",
    # Packed fp32 instructions are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the library; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        _run([cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    out = os.path.join(LIBDIR, LIBNAME)
    tmp = out + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

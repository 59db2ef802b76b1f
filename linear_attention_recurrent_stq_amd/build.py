"""Build the HIP library in-tree: ``libstq.so`` next to this file (gfx950 only).

Each source is compiled to an object of its own (in parallel, under
``_build/``) and the objects are linked into the shared library.  With
``debug_validate=True`` the same sources are built with STQ_DEBUG_VALIDATE
into ``libstq_debug.so``: every call that takes slot ids then copies them to
the host and rejects duplicates and out-of-range ids before any launch.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libstq.so")
LIB_DEBUG = os.path.join(HERE, "libstq_debug.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = [os.path.join(HERE, "csrc", f)
           for f in ("stq_host.cpp", "stq_alloc.cpp", "stq_kernels.hip", "stq_window.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # reproducible fp32: no contraction, correctly rounded division, denormals kept
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    # no packed-fp32 instructions in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # occupancy targets are hints; head sizes that cannot meet them keep fewer waves
    "-Wno-pass-failed",
]


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n, len(SOURCES)))


def build(verbose: bool = False, debug_validate: bool = False) -> str:
    """Compile every source and link the library (always recompiles)."""
    tag = "debug" if debug_validate else "release"
    objdir = os.path.join(OBJDIR, tag)
    os.makedirs(objdir, exist_ok=True)
    extra = ["-DSTQ_DEBUG_VALIDATE=1"] if debug_validate else []
    inc = ["-I", os.path.join(ROOT, "include")]

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *extra, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        return obj

    with ThreadPoolExecutor(_jobs()) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    out = LIB_DEBUG if debug_validate else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, debug_validate="--debug-validate" in sys.argv)
    print(LIB_DEBUG if "--debug-validate" in sys.argv else LIB)

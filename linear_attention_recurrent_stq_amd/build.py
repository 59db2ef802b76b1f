"""Build the HIP library in-tree: ``libstq.so`` next to this file (gfx950 only).

Each source is compiled to an object of its own (in parallel, under
``_build/``) and the objects are linked into the shared library.  The same
kernels are also linked with the host source built with STQ_DEBUG_VALIDATE
into ``libstq_debug.so``: there every call that takes slot ids copies them to
the host and rejects duplicates and out-of-range ids before any launch.

``build_sanitized()`` links the same kernels with the host sources built with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; the device
code is the release code) into ``libstq_san.so``, for the CPU test suite run
by ``tests/sanitize.sh``.
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
LIB_SAN = os.path.join(HERE, "libstq_san.so")
# host-only sanitizer flags (each -fsanitize= behind -Xarch_host: no GPU code is built with it)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
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
    return max(1, min(16, n, len(SOURCES) + 1))


def build(verbose: bool = False) -> str:
    """Compile every source and link libstq.so and libstq_debug.so (always
    recompiles).  Returns the path of libstq.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    host = SOURCES[0]
    jobs = [(src, os.path.join(OBJDIR, os.path.basename(src) + ".o"), []) for src in SOURCES]
    jobs.append((host, os.path.join(OBJDIR, "debug_" + os.path.basename(host) + ".o"),
                 ["-DSTQ_DEBUG_VALIDATE=1"]))

    def compile_one(job):
        src, obj, extra = job
        cmd = [HIPCC, *FLAGS, *extra, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        return obj

    # the largest source first, so the others compile beside it
    order = sorted(jobs, key=lambda j: -os.path.getsize(j[0]))
    with ThreadPoolExecutor(_jobs()) as ex:
        list(ex.map(compile_one, order))
    objs = [j[1] for j in jobs]
    for out, use in ((LIB, objs[:len(SOURCES)]), (LIB_DEBUG, [objs[-1]] + objs[1:len(SOURCES)])):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *use, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """libstq_san.so: host sources with ASan + UBSan, kernels as in the release
    build (build() must have run).  Load it with clang's shared ASan runtime
    preloaded (tests/sanitize.sh)."""
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = []
    for src in SOURCES:
        if src.endswith(".hip"):
            objs.append(os.path.join(OBJDIR, os.path.basename(src) + ".o"))
            continue
        obj = os.path.join(OBJDIR, "san_" + os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, "-O1", *SAN, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB_SAN + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libasan", *SAN, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_SAN)
    return LIB_SAN


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        build(verbose="-v" in sys.argv)
        print(LIB, LIB_DEBUG)

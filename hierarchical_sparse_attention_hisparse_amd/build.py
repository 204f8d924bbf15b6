"""Build the libraries in-tree for gfx950 with hipcc (no JIT, no cache).

libhisparse.so is the library.  libhisparse_diag.so is the same sources with
the plan kernel's phase trace compiled in (HISPARSE_PHASE_TRACE) plus the
floor kernels of diag.hip; it exports the entry points of include/hisparse.h
and of include/hisparse_diag.h.  Objects are compiled in parallel in a
temporary folder and linked into both libraries."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhisparse.so")
DIAG_LIB = os.path.join(HERE, "libhisparse_diag.so")
SOURCES = ["abi.hip", "resolve.hip", "gather.hip", "mla_decode.hip", "maintain.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _compile_all(jobs, verbose):
    """jobs: [(source, object, extra flags)], compiled in parallel."""
    procs = []
    for src, obj, extra in jobs:
        cmd = [hipcc()] + HIPCC_FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
    failed = [cmd for cmd, pr in procs if pr.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])


def _link(objs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build_library(force: bool = True, verbose: bool = False) -> str:
    if not force and os.path.exists(LIB) and os.path.exists(DIAG_LIB):
        return LIB
    tmpdir = tempfile.mkdtemp(prefix="hisparse_build_")
    try:
        obj = lambda name: os.path.join(tmpdir, name + ".o")
        jobs = [(s, obj(s[:-4]), []) for s in SOURCES]
        jobs.append(("resolve.hip", obj("resolve_trace"), ["-DHISPARSE_PHASE_TRACE"]))
        jobs.append(("diag.hip", obj("diag"), ["-DHISPARSE_PHASE_TRACE"]))
        _compile_all(jobs, verbose)
        _link([obj(s[:-4]) for s in SOURCES], LIB, verbose)
        diag_objs = [obj("resolve_trace") if s == "resolve.hip" else obj(s[:-4]) for s in SOURCES]
        _link(diag_objs + [obj("diag")], DIAG_LIB, verbose)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    build_library(force=True, verbose="-v" in sys.argv)
    print(LIB)
    print(DIAG_LIB)

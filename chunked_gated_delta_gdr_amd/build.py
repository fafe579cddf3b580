"""Build libgdr.so (all HIP sources of the library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgdr.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is harmless
    noise = "is not a recognized feature for this target"
    return res.returncode, [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    """Compile every source to an object (in parallel: each holds its own kernels and their
    launchers, so no device code crosses files), then link the shared library."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = out + ".tmp"
    objdir = tempfile.mkdtemp(prefix="gdr_build_")
    try:
        jobs = []
        for src in sources():
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            jobs.append((src, obj, [hipcc, *HIPCC_FLAGS, *extra, "-c", "-I", os.path.join(ROOT, "include"),
                                    "-I", os.path.join(PKG, "csrc"), src, "-o", obj]))
        if verbose:
            for _, _, cmd in jobs:
                print(" ".join(cmd), flush=True)
        workers = max(1, min(len(jobs), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            results = list(pool.map(lambda j: _run(j[2]), jobs))
        msgs = [m for _, ms in results for m in ms]
        if any(rc != 0 for rc, _ in results):
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
        link = [hipcc, *HIPCC_FLAGS, *extra, *[o for _, o, _ in jobs], "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, lmsgs = _run(link)
        if rc != 0:
            raise RuntimeError("link failed:\n" + "\n".join(lmsgs))
        msgs += lmsgs
        if verbose and msgs:
            print("\n".join(msgs))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libmxq.so (all HIP sources of the package) for gfx950 with hipcc.

The library records a hash of the sources, the public header and the compiler
flags it was built from (``mxq_build_id()``); the binding compares it with
``source_hash()`` of the tree at load time and refuses a library built from
other sources, so a test or benchmark never runs a stale binary.
"""
from __future__ import annotations

import glob
import hashlib
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmxq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -fno-gpu-flush-denormals-to-zero: the encoders rely on fp32 subnormals.
# -ffp-contract=off: each fp32 product/quotient the method defines rounds once.
# packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 are generated.
HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def dependencies():
    """Every file whose content goes into the library."""
    return sources() + sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + [
        os.path.join(INCLUDE, "mxq.h")]


def source_hash() -> str:
    """sha256 (first 16 hex digits) over the flags and the name and content of
    every dependency."""
    h = hashlib.sha256(" ".join(HIPFLAGS).encode())
    for p in dependencies():
        h.update(os.path.relpath(p, ROOT).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link one shared library
    (always recompiles)."""
    ident = source_hash()
    flags = [*HIPFLAGS, f"-DMXQ_BUILD_ID=\"{ident}\"", "-I", INCLUDE, "-I", CSRC]
    tmpdir = tempfile.mkdtemp(prefix="mxq_build_")
    try:
        jobs = []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            jobs.append(([HIPCC, *flags, "-c", src, "-o", obj], obj))

        def run(job):
            cmd, _ = job
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)

        with ThreadPoolExecutor(max_workers=max(1, min(len(jobs), os.cpu_count() or 1))) as ex:
            list(ex.map(run, jobs))
        tmp = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o in jobs],
                "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


def stale() -> bool:
    """True when libmxq.so is missing or older than a source or the header."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in dependencies())


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

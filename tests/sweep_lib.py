"""Build and load tests/libcvt_sweep.so, the test-only HIP library that runs
the product's fp32 -> E4M3 / E2M1 / bf16 converters over runs of fp32 bit
patterns (tests/csrc/cvt_sweep.hip).  Built by __graft_entry__.build() with
the product library's compiler flags; the build id (a hash of the sources and
flags) is checked at load, so a stale build is refused."""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
SRC = os.path.join(HERE, "csrc", "cvt_sweep.hip")
LIB = os.path.join(HERE, "libcvt_sweep.so")


def _deps():
    from block_scaled_precision_mxfp8_amd import build as pb
    return pb, [SRC, os.path.join(pb.CSRC, "mxq_device.hpp")]


def source_hash() -> str:
    pb, deps = _deps()
    h = hashlib.sha256(" ".join(pb.HIPFLAGS).encode())
    for p in deps:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def build() -> str:
    pb, _ = _deps()
    tmp = LIB + ".tmp"
    subprocess.run([pb.HIPCC, *pb.HIPFLAGS, "-shared", f"-DSWEEP_BUILD_ID=\"{source_hash()}\"",
                    "-I", pb.CSRC, SRC, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


def load() -> ctypes.CDLL:
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    L.cvt_sweep_build_id.restype = ctypes.c_char_p
    if L.cvt_sweep_build_id().decode() != source_hash():
        raise RuntimeError(f"{LIB} was built from other sources (run __graft_entry__.build())")
    for nm in ("cvt_sweep_e4m3", "cvt_sweep_e2m1", "cvt_sweep_bf16"):
        fn = getattr(L, nm)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p,
                       ctypes.c_void_p, ctypes.c_void_p]
    return L

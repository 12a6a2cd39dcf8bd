"""Build libmxq.so (all HIP sources of the package) for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

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
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into one shared library (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *HIPFLAGS, "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    """True when libmxq.so is missing or older than a source or the header."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + glob.glob(os.path.join(CSRC, "*.hpp")) + [os.path.join(INCLUDE, "mxq.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

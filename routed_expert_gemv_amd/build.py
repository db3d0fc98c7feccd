"""Build libmoe_decode.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_decode.so")
SOURCES = [os.path.join(CSRC, "moe_kernels.hip"), os.path.join(CSRC, "moe_prefill.hip"),
           os.path.join(CSRC, "moe_abi.cpp")]
HEADERS = [os.path.join(CSRC, "moe_internal.h"), os.path.join(INCLUDE, "moe_decode.h"),
           os.path.join(INCLUDE, "moe_prefill.h")]
ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for every HIP file of this library.
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile the HIP sources into LIB (always when force, else only if stale)."""
    if not force and not stale():
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I" + INCLUDE, "-I" + CSRC] + SOURCES + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (r.returncode, " ".join(cmd), r.stderr))
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))

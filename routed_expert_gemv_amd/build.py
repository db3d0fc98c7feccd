"""Build libmoe_decode.so (gfx950) in-tree with hipcc.

The library carries the SHA-256 of the sources it was built from (exported as
moe_build_id); the loader refuses a library whose id differs from the
sources in the tree, so a test never runs an old binary by accident.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_decode.so")
SOURCES = [os.path.join(CSRC, "moe_kernels.hip"), os.path.join(CSRC, "moe_layer1.hip"),
           os.path.join(CSRC, "moe_prefill.hip"), os.path.join(CSRC, "moe_noalloc.hip"),
           os.path.join(CSRC, "moe_abi.cpp")]
HEADERS = [os.path.join(CSRC, "moe_internal.h"), os.path.join(CSRC, "moe_device.h"),
           os.path.join(INCLUDE, "moe_decode.h"), os.path.join(INCLUDE, "moe_prefill.h")]
ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for every HIP file of this library.
# Kernel arguments are preloaded into SGPRs at dispatch (up to 16 dwords; the
# compiler keeps a loader in front of each kernel for firmware that does not
# preload): a kernel's first loads then need not wait for its arguments.
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
               "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-kernarg-preload-count=16"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def source_id() -> str:
    """SHA-256 (hex) over the compiler flags and the names and contents of the
    sources and headers."""
    h = hashlib.sha256()
    h.update(" ".join(HIPCC_FLAGS).encode() + b"\0")
    for path in sorted(SOURCES + HEADERS):
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()


def stale() -> bool:
    """True when LIB is missing or older than a source (mtime; the loader's
    content check is the authoritative one)."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


# moe_kernels.hip is compiled once per part (-DMOE_PART): part 0 holds the
# entry points and dispatch, parts 1..8 the kernels of hidden width 512*part,
# parts 9..21 the down-projection kernels of one lane mapping each.
KERNEL_PARTS = 22


def _units():
    """(source, extra flags, object name) of every translation unit."""
    units = []
    for src in SOURCES:
        base = os.path.splitext(os.path.basename(src))[0]
        if base == "moe_kernels":
            units += [(src, ["-DMOE_PART=%d" % p], "%s_p%02d.o" % (base, p))
                      for p in range(KERNEL_PARTS)]
        else:
            units.append((src, [], base + ".o"))
    return units


def build(force: bool = True, verbose: bool = False, jobs: int = 0) -> str:
    """Compile the HIP sources into LIB (always when force, else only if stale):
    every translation unit in parallel (jobs, default: the CPUs this process
    may use), then one link."""
    if not force and not stale():
        return LIB
    import concurrent.futures
    import tempfile

    jobs = jobs or max(1, len(os.sched_getaffinity(0)))
    common = [hipcc()] + HIPCC_FLAGS + ['-DMOE_BUILD_ID="%s"' % source_id(), "-I" + INCLUDE,
                                       "-I" + CSRC]
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmpdir:
        def compile_unit(u):
            src, extra, obj = u
            out = os.path.join(tmpdir, obj)
            cmd = common + extra + ["-c", src, "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            return cmd, r, out

        # the largest units first, so that the pool drains evenly
        units = sorted(_units(), key=lambda u: 0 if "MOE_PART" in "".join(u[1]) else 1)
        objs = []
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for cmd, r, out in ex.map(compile_unit, units):
                if r.returncode != 0:
                    raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (r.returncode, " ".join(cmd),
                                                                        r.stderr))
                if verbose:
                    sys.stderr.write(r.stderr)
                objs.append(out)
        tmp = LIB + ".tmp%d" % os.getpid()
        # -z defs: a part that fails to define what another part calls is a
        # link error here, not a load failure later
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,-z,defs"] + objs + \
            ["-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed (%d):\n%s\n%s" % (r.returncode, " ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))

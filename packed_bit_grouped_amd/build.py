"""Build libmoe_w4.so in place with hipcc for gfx950.

Usage: python -m packed_bit_grouped_amd.build [-j N] [--host-check OUT.so]
                                               [--stamps OUT.so]
Every call recompiles every source (the build check wants a real compile).
--host-check also builds a copy of the library whose host code at the C ABI
(argument checks, workspace carving, launch set-up: api.cpp and the entry
points of noalloc.hip and probe.hip) carries AddressSanitizer and
UndefinedBehaviorSanitizer; device code is not instrumented.  It is for
CPU-side checks only (load it with the ASan runtime preloaded).
--stamps also builds a copy whose decode kernels write phase clock stamps
(MOE_DEC_STAMPS; moe_dbg_dec_stamps names the buffer), for the timeline
measurement only.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libmoe_w4.so")
SOURCES = ["api.cpp", "route_permute.hip", "quant_combine.hip",
           "proj_gemv.hip", "proj_decode.hip", "proj_m16.hip",
           "proj_mfma8.hip", "noalloc.hip", "probe.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 VALU forms are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
         f"-I{INCLUDE}"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, objdir: str) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
    if r.stderr.strip():
        sys.stderr.write(r.stderr)
    return obj


# sources whose host code is instrumented in the host-check build
HOST_CHECK_SOURCES = ["api.cpp", "noalloc.hip", "probe.hip"]
# host-side sanitizers only: each flag goes to the host compilation
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_check(out: str, jobs: int = 0) -> str:
    """The library with sanitized host code at the ABI (see the module
    docstring); the kernel sources' objects come from the regular build
    (built first if missing)."""
    objdir = os.path.join(HERE, "_build")
    plain = [s for s in SOURCES if s not in HOST_CHECK_SOURCES]
    if not all(os.path.exists(os.path.join(objdir, s + ".o")) for s in plain):
        build(jobs, verbose=False)
    sandir = os.path.join(objdir, "host_check")
    os.makedirs(sandir, exist_ok=True)

    def comp(src):
        obj = os.path.join(sandir, src + ".o")
        flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", *SAN_FLAGS]
        r = subprocess.run([hipcc(), "-x", "hip", *flags, "-c", os.path.join(CSRC, src), "-o",
                            obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
        return obj

    with ThreadPoolExecutor(max_workers=jobs or len(HOST_CHECK_SOURCES)) as ex:
        objs = list(ex.map(comp, HOST_CHECK_SOURCES))
    objs += [os.path.join(objdir, s + ".o") for s in plain]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS[:4],
           "-Xarch_host", "-shared-libsan", "-o", out, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    return out


def build_stamps(out: str, jobs: int = 0) -> str:
    """The library with the decode kernels' phase stamps compiled in; the
    other sources' objects come from the regular build (built first if
    missing)."""
    objdir = os.path.join(HERE, "_build")
    plain = [s for s in SOURCES if s != "proj_decode.hip"]
    if not all(os.path.exists(os.path.join(objdir, s + ".o")) for s in plain):
        build(jobs, verbose=False)
    sdir = os.path.join(objdir, "stamps")
    os.makedirs(sdir, exist_ok=True)
    obj = os.path.join(sdir, "proj_decode.hip.o")
    r = subprocess.run([hipcc(), "-x", "hip", *FLAGS, "-DMOE_DEC_STAMPS", "-c",
                        os.path.join(CSRC, "proj_decode.hip"), "-o", obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for proj_decode.hip:\n{r.stderr[-8000:]}")
    objs = [obj] + [os.path.join(objdir, s + ".o") for s in plain]
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    return out


def build(jobs: int = 0, verbose: bool = True) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=0)
    ap.add_argument("--host-check", metavar="OUT", default=None)
    ap.add_argument("--stamps", metavar="OUT", default=None)
    a = ap.parse_args()
    build(a.j)
    if a.host_check:
        print(f"built {build_host_check(a.host_check, a.j)}")
    if a.stamps:
        print(f"built {build_stamps(a.stamps, a.j)}")

"""Compile libgc.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m two_point_angular_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libgc.so")
BINDIR = os.path.join(PKG, "bin")
CLI = os.path.join(BINDIR, "galaxy_gc")
ARCH = "gfx950"

# -packed-fp32-ops: no packed FP32 (v_pk_*_f32) instructions anywhere in the device code.
# pragma-unroll-threshold: the bin-table kernel's matrix-core loop (32 tiles, each with its rare
# drain paths) must unroll fully, which the default size threshold refuses.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-pragma-unroll-threshold=100000",
             "-I", os.path.join(ROOT, "include")]

SOURCES = ["gc_kernels.hip", "gc_api.cpp", "gc_ceilings.hip", "gc_ladder.hip", "gc_io.cpp"]
CLI_SOURCE = "galaxy_gc.cpp"   # the end-to-end program, linked against libgc.so


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libgc.so failed")
    os.replace(tmp, LIB)
    build_cli(verbose)
    return LIB


def build_cli(verbose: bool = False) -> str:
    """galaxy_gc (bin/), linked against lib/libgc.so through an $ORIGIN-relative rpath."""
    os.makedirs(BINDIR, exist_ok=True)
    tmp = CLI + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIP_FLAGS, "-x", "hip", os.path.join(CSRC, CLI_SOURCE), "-o", tmp, "-L", LIBDIR, "-lgc",
           "-Wl,-rpath,$ORIGIN/../lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build of galaxy_gc failed")
    os.replace(tmp, CLI)
    return CLI


if __name__ == "__main__":
    print(build(verbose=True))

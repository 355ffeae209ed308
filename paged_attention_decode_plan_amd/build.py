"""Build libpa.so (gfx950) in-tree with hipcc."""

from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = ["pa_plan.cpp", "pa_kernels.hip", "pa_stream.hip", "pa_static.hip", "pa_indexer.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 are generated.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def source_sha() -> str:
    """Short hash of the library's sources: ties a counter run to the code it
    measured."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f in SOURCES or f.endswith(".h"):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


CEILING_LIB = os.path.join(PKG, "libpa_ceiling.so")


def build_ceiling(verbose: bool = False) -> str:
    """The read-only bandwidth probes of bench.py --ceiling (a measurement
    tool in a library of its own; libpa.so does not contain it)."""
    tmp = CEILING_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, os.path.join(CSRC, "pa_ceiling.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libpa_ceiling.so")
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


def build_library(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link libpa.so."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    procs = []
    for s in SOURCES:
        obj = os.path.join(objdir, s + ".o")
        cmd = [HIPCC, *compile_flags, "-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = False
    for _, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out + err)
            failed = True
    if failed:
        raise RuntimeError("hipcc failed compiling libpa.so sources")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in procs], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libpa.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_ceiling(verbose=True))

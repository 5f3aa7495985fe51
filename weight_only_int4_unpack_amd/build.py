"""Build ``libw4a16.so`` (gfx950) in-tree with hipcc.

Usage: ``python -m weight_only_int4_unpack_amd.build`` or ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libw4a16.so")
# measurement probe for bench.py (a plain streaming read), its own library
PROBE_LIB = os.path.join(PKG, "libw4a16_probe.so")

ARCH = "gfx950"
# Packed fp32 ops stay off: hipcc still emits v_pk_* f16 ops, which are
# what the dequantisation uses.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
SOURCES = ["w4a16_host.cpp", "w4a16_kernels.hip", "w4a16_noalloc.hip"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libw4a16.so)")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library."""
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *HIP_FLAGS, *lang, "-I", os.path.join(ROOT, "include"), "-c",
               os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    tmp = PROBE_LIB + ".tmp"
    _run([cc, *HIP_FLAGS, "-x", "hip", "-shared", os.path.join(CSRC, "probe_read.hip"),
          "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libep.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m combine_moe_layout_amd.build``; ``__graft_entry__.build()``
calls :func:`build_library`.  Objects go to ``_build/`` at the repo root; the
library lands next to this file, where the binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libep.so")
SOURCES = ["ep_api.hip", "ep_layout.hip", "ep_dispatch.hip", "ep_fused.hip", "ep_combine.hip",
           "ep_group.hip", "ep_aux.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # IEEE fp32 division: the FP8 scale and its reciprocal are single correctly
    # rounded divisions, bit-identical to any IEEE implementation.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep fp32 denormals (no flush to zero)
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build_library(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libep.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, r.stderr))
        # the host pass does not know the packed-fp32 feature; that warning is expected
        noise = [ln for ln in r.stderr.splitlines()
                 if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
        if verbose and noise:
            print("\n".join(noise), flush=True)
        return obj

    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))

"""Build libep.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m combine_moe_layout_amd.build``; ``__graft_entry__.build()``
calls :func:`build_library`.  ``python -m combine_moe_layout_amd.build
--resources`` prints each kernel's registers, LDS, scratch and occupancy as
the compiler reports them for gfx950.  Objects go to ``_build/`` at the repo root; the
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
           "ep_group.hip", "ep_scales.hip", "ep_aux.hip"]

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


_FIELDS = (("VGPRs", "vgpr"), ("AGPRs", "agpr"), ("TotalSGPRs", "sgpr"),
           ("ScratchSize [bytes/lane]", "scratch"), ("LDS Size [bytes/block]", "lds"),
           ("Occupancy [waves/SIMD]", "occupancy"), ("VGPRs Spill", "vgpr_spill"),
           ("SGPRs Spill", "sgpr_spill"))


def resource_usage() -> list:
    """Per-kernel register, LDS and scratch use of the gfx950 build, read from
    the compiler's kernel-resource-usage remarks (one dict per kernel: mangled
    name, source file and the fields in ``_FIELDS``)."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def one(src: str) -> list:
        obj = os.path.join(BUILD, "ru_" + src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, "--offload-device-only", "-Rpass-analysis=kernel-resource-usage",
               "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, r.stderr))
        rows, cur = [], None
        for ln in r.stderr.splitlines():
            if "remark:" not in ln:
                continue
            body = ln.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
            key, _, val = body.partition(":")
            key, val = key.strip(), val.strip()
            if key == "Function Name":
                cur = {"kernel": val, "source": src}
                rows.append(cur)
            elif cur is not None:
                for label, name in _FIELDS:
                    if key == label:
                        cur[name] = int(val)
        return rows

    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        return [row for rows in ex.map(one, SOURCES) for row in rows]


def _demangle(names: list) -> list:
    for tool in ("/opt/rocm/llvm/bin/llvm-cxxfilt", shutil.which("c++filt")):
        if tool and os.path.exists(tool):
            r = subprocess.run([tool], input="\n".join(names), capture_output=True, text=True)
            if r.returncode == 0:
                return r.stdout.splitlines()
    return names


if __name__ == "__main__":
    if "--resources" in sys.argv:
        rows = resource_usage()
        names = _demangle([r["kernel"] for r in rows])
        print("| kernel | source | VGPR | AGPR | SGPR | LDS B | scratch B/lane | waves/SIMD | spills |")
        print("|---|---|---:|---:|---:|---:|---:|---:|---:|")
        for r, n in zip(rows, names):
            n = n.replace("ep::", "").split("(")[0]
            print("| `%s` | %s | %d | %d | %d | %d | %d | %d | %d |" % (
                n, r["source"], r.get("vgpr", -1), r.get("agpr", -1), r.get("sgpr", -1), r.get("lds", -1),
                r.get("scratch", -1), r.get("occupancy", -1), r.get("vgpr_spill", 0) + r.get("sgpr_spill", 0)))
    else:
        print(build_library(verbose="-v" in sys.argv))

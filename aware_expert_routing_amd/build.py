"""Build libmoe_decode.so in-tree with hipcc for gfx950.

Usage: python -m aware_expert_routing_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_decode.so")
SOURCES = ["router.hip", "select.hip", "route_select.hip", "ffn.hip", "stream.hip", "static_scratch.hip",
           "api.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Measurement library: the same sources with the expert FFN's phase stamps
# compiled in (MOE_PHASE_STAMPS); bench.py --phase-timeline loads it. The
# product library never contains them.
PHASES_LIB = os.path.join(PKG, "libmoe_decode_phases.so")
PHASES_DEFINE = "-DMOE_PHASE_STAMPS"


def _compile(src: str, defines=()) -> str:
    tag = "_phases" if defines else ""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, *defines, *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link the shared library, and the
    measurement library (the expert FFN with phase stamps). Returns the
    product library's path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, ()) for src in SOURCES] + [("ffn.hip", (PHASES_DEFINE,))]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    product = objs[:len(SOURCES)]
    _link(product, LIB)
    phases = [o for o, src in zip(product, SOURCES) if src != "ffn.hip"] + [objs[-1]]
    _link(phases, PHASES_LIB)
    if verbose:
        print(f"built {LIB} and {PHASES_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

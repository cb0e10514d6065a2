"""Builds librra.so (HIP, gfx950) in-tree from csrc/.

Each source is compiled to an object under _build/ in parallel, then linked.
Usage: python quantized_gemv_flash_amd/build.py [--force]  (a plain script: importing
the package would load the library it builds)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librra.so")
SOURCES = ["gemv.hip", "attention.hip", "elementwise.hip", "model.cpp"]
HEADERS = [os.path.join(CSRC, h) for h in ("rra_internal.h", "frag.h", "epilogue.h")] + [
    os.path.join(INCLUDE, "rra.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-source extra flags: the GEMV keeps MFMA accumulators in ordinary VGPRs,
# so the per-block scale FMAs read them without v_accvgpr_read copies.
EXTRA = {"gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    dep = max([os.path.getmtime(path)] + [os.path.getmtime(h) for h in HEADERS])
    if os.path.exists(obj) and os.path.getmtime(obj) >= dep and os.environ.get("RRA_REBUILD") != "1":
        return obj
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(force: bool = False) -> str:
    """Compile every HIP source for gfx950 and link librra.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    if force:
        os.environ["RRA_REBUILD"] = "1"
    try:
        with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            objs = list(ex.map(_compile, SOURCES))
    finally:
        if force:
            os.environ.pop("RRA_REBUILD", None)
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))

"""Builds libzero_mi355x.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzero_mi355x.so")

SOURCES = ["status.cpp", "plan.cpp", "pieces.cpp", "schedule.cpp", "offload.cpp", "adamw.hip", "reduce.hip",
           "gather.hip"]

# -ffp-contract=off: the AdamW and reduction arithmetic is specified operation
# by operation; no multiply-add fusion. Packed fp32 instructions are disabled.
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-ffp-contract=off", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


def _compile(src: str, obj: str, defines: List[str], save_temps: Optional[str]) -> List[str]:
    if src.endswith(".hip"):
        cmd = ["hipcc", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + defines + DEVICE
        if save_temps:
            cmd += [f"-save-temps={'obj'}"]
    else:
        # host-only C++ (no device code): compiled as plain C++ against the HIP runtime API;
        # no errno from sqrtf, so the host AdamW loop vectorizes (IEEE results unchanged)
        rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
        cmd = (["hipcc", "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + defines +
               [f"-I{rocm}/include", "-D__HIP_PLATFORM_AMD__", "-fno-math-errno"])
    return cmd


def build(out: str = LIB, defines: Optional[List[str]] = None, save_temps: Optional[str] = None,
          verbose: bool = False, objdir: Optional[str] = None) -> str:
    """Compile every source and link the shared library; returns its path."""
    defines = list(defines or [])
    objdir = save_temps or objdir or os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append(_compile(src, obj, defines, save_temps))

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, cwd=objdir)

    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(run, cmds))
    tmp = out + ".tmp"
    link = ["hipcc", "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    run(link)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    # python _build.py [-v] [-D NAME=VALUE ...] [-o OUT]: OUT defaults to the product
    # library; a build with switches (-D) for a measured comparison goes elsewhere,
    # loaded through the ZERO_MI355X_LIB environment variable.
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("-D", action="append", default=[], metavar="NAME=VALUE")
    ap.add_argument("-o", default=LIB)
    a = ap.parse_args()
    out = os.path.abspath(a.o)
    objdir = None
    if out != LIB:
        objdir = os.path.join(ROOT, "_build", "variant_" + os.path.splitext(os.path.basename(out))[0])
    build(out, defines=[f"-D{d}" for d in a.D], objdir=objdir, verbose=a.v)

"""Compile liboccult.so (HIP C++ for gfx950) in-tree.

    python expert_top_router_amd/build.py

(run by path: importing the package loads the library this script builds).

Every source is compiled with hipcc for gfx950 only; packed-fp32 instructions
are disabled in device code (hipcc's host pass warns that it does not know
that feature, which is harmless).
"""
from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "occult")
LIB = os.path.join(PKG, "liboccult.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["occ_api.cpp", "occ_route.hip", "occ_route_filter.hip", "occ_route_mfma.hip", "occ_brim.hip", "occ_permute.hip", "occ_coact.hip",
           "occ_affinity.hip", "occ_backward.hip", "occ_gemm.hip", "occ_gemm_bwd.hip",
           "occ_bwd_f32.hip"]

FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *lang, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Wl,-z,defs",
                           "-o", tmp, *objs])
    # every symbol must resolve now (a kernel whose host stub was not emitted
    # shows up here, not at the first launch)
    ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

"""Build libmoegg.so in-tree with hipcc for gfx950.

    python -m moe_grouped_block_amd.build

Compiles every source under ``csrc/`` each time it is called (objects in
parallel) and links ``moe_grouped_block_amd/libmoegg.so``.  No GPU is needed:
hipcc cross-compiles for gfx950.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoegg.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    # registers stay registers: no promotion of private arrays into LDS
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]
SOURCES = ["moegg_api.cpp", "moegg_kernels.hip", "inst_e4m3.hip", "inst_e2m1.hip", "inst_bf16.hip", "inst_e5m2.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()

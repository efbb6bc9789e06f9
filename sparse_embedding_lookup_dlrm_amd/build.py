"""Build libdlrm_embbag.so in-tree with hipcc for gfx950.

    python -m sparse_embedding_lookup_dlrm_amd.build          # build (always recompiles)
    python -m sparse_embedding_lookup_dlrm_amd.build --asm    # also write gfx950 assembly to _build/

Each source compiles to its own object in parallel, then one shared library is
linked next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdlrm_embbag.so")

SOURCES = ["embbag_fwd.hip", "embbag_bwd.hip", "offsets.hip", "noalloc.hip", "probe.hip", "api.cpp"]
ARCH = "gfx950"

# Packed fp32 instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build libdlrm_embbag.so)")
    return p


def _compile(src: str, asm: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if asm and src.endswith(".hip"):
        s = os.path.join(BUILD, os.path.splitext(src)[0] + f"-{ARCH}.s")
        cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "--cuda-device-only", "-S",
               path, "-o", s]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"asm failed: {r.stderr}")
    return obj


def build(asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    args = ap.parse_args()
    build(asm=args.asm, verbose=True)
    sys.exit(0)

"""Build the gfx950 HIP library ``libnvfp4.so`` in-tree.

    python -m bit_block_scaled_amd.build        # or bit_block_scaled_amd.build.build()

Each source compiles to an object under ``bit_block_scaled_amd/_build`` (in
parallel), then hipcc links them into ``bit_block_scaled_amd/lib/libnvfp4.so``.
Every call recompiles.  Packed-FP32 instruction selection is disabled for all
device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libnvfp4.so")

# The GEMM's tile shapes are separate units (the slowest to compile), listed first.
SOURCES = ["gemm_tile_4x4.hip", "gemm_tile_4x3.hip", "gemm_tile_3x4.hip", "gemm_tile_4x2.hip",
           "gemm_tile_2x4.hip", "gemm_tile_2x2.hip", "attention.hip", "rht.hip", "quantize.hip", "gemm.hip", "kv.hip", "smooth.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the NVFP4 library)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"          # the host pass does not know the device feature
    err = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    workers = max(1, min(8, len(SOURCES), os.cpu_count() or 4))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)

"""Build libbiloco_hip.so in-tree with hipcc for gfx950 (no JIT cache).

Usage: python -m bit_weight_gemm_amd.build   (or __graft_entry__.build()).
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbiloco_hip.so")

SOURCES = ["biloco_api.cpp", "k_prep.hip", "k_unfused.hip", "k_fused_gemv.hip", "k_fused_mfma.hip",
           "k_composed.hip", "k_peel.hip", "scratch.hip"]
HEADERS = ["biloco_device.h", "biloco_internal.h", os.path.join("..", "..", "include", "biloco.h")]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed fp32 vector ops are switched off for every device compile.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # a lone lane's fetch-add must not be rewritten into a wave-wide
          # aggregate that waits for the result at once
          "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + list(extra) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr}")
    return obj


FLOOR_SRC = os.path.join(PKG, "floor", "stream_floor.hip")
FLOOR_LIB = os.path.join(PKG, "libbiloco_floor.so")


def build_floor(verbose: bool = True) -> str:
    """The measurement-only read/empty kernels bench.py's stream-floor leg
    times (a library of their own, not part of libbiloco_hip)."""
    tmp = FLOOR_LIB + ".tmp"
    cmd = [HIPCC] + COMMON + ["-shared", "-x", "hip", FLOOR_SRC, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {FLOOR_SRC}:\n{p.stderr}")
    os.replace(tmp, FLOOR_LIB)
    if verbose:
        print(f"built {FLOOR_LIB}")
    return FLOOR_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


TL_BUILD = os.path.join(PKG, "_build_tl")
TL_LIB = os.path.join(PKG, "libbiloco_tl.so")


def build_timeline(verbose: bool = True) -> str:
    """The same library compiled with BILOCO_TIMELINE: the product kernels
    also write per-wave stamps of the real-time counter, which bench.py's
    --timeline leg reads (a measurement build; never the product path)."""
    os.makedirs(TL_BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, TL_BUILD, ["-DBILOCO_TIMELINE"]), srcs))
    tmp = TL_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, TL_LIB)
    if verbose:
        print(f"built {TL_LIB}")
    return TL_LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

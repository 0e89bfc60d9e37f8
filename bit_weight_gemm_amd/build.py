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


RESOURCES = os.path.join(BUILD, "resource_usage.json")


def _resources(stderr: str) -> dict:
    """Per-kernel VGPRs and scratch bytes per lane from hipcc's
    -Rpass-analysis=kernel-resource-usage remarks."""
    out, name = {}, None
    for line in stderr.splitlines():
        if "Function Name: " in line:
            name = line.split("Function Name: ", 1)[1].split(" [")[0].strip()
            out[name] = {}
        elif name and "VGPRs: " in line:
            out[name]["vgprs"] = int(line.split("VGPRs: ", 1)[1].split()[0])
        elif name and "ScratchSize [bytes/lane]: " in line:
            out[name]["scratch_bytes_per_lane"] = int(line.split("ScratchSize [bytes/lane]: ", 1)[1].split()[0])
    return out


def _compile(src: str, build_dir: str = BUILD, extra=(), usage: dict | None = None) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + list(extra) + ["-Rpass-analysis=kernel-resource-usage", "-x", "hip",
                                            "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr}")
    if usage is not None:
        usage[src] = _resources(p.stderr)
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
    usage: dict = {}
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, BUILD, (), usage), srcs))
    # the kernels' register use, for tests/test_build_resources.py
    import json
    with open(RESOURCES, "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
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

"""ctypes view of the fp64 CPU oracle (``biloco_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only users.  The HIP library never
imports, loads or calls anything in this package, and this package never
touches the HIP library.

Each wrapper takes numpy arrays in the layouts documented in the C file and
returns numpy arrays; the C routines are the plain definitions (see the
header of ``biloco_oracle.c`` for the passages they follow).  The sign
peeling decomposition is plain numpy in ``peel.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "biloco_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_biloco.so")
# a build of the same source made elsewhere (the sanitized one of the tests)
_LIB_OVERRIDE = os.environ.get("BILOCO_ORACLE_LIB")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP over independent outputs)."""
    if _LIB_OVERRIDE:
        return _LIB_OVERRIDE
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        d, u, i64, p = ctypes.c_double, ctypes.c_uint, ctypes.c_int64, ctypes.c_void_p
        lib.oracle_e2m1_value.restype = d
        lib.oracle_e2m1_value.argtypes = [u]
        lib.oracle_e4m3_value.restype = d
        lib.oracle_e4m3_value.argtypes = [u]
        lib.oracle_e4m3_encode.restype = u
        lib.oracle_e4m3_encode.argtypes = [d]
        lib.oracle_e2m1_encode.restype = u
        lib.oracle_e2m1_encode.argtypes = [d, d]
        lib.oracle_e2m1_encode_n.restype = None
        lib.oracle_e2m1_encode_n.argtypes = [p, p, i64, p]
        lib.oracle_e4m3_encode_n.restype = None
        lib.oracle_e4m3_encode_n.argtypes = [p, i64, p]
        lib.oracle_bf16_value.restype = d
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_quant_act_fp4.restype = None
        lib.oracle_quant_act_fp4.argtypes = [p, i64, i64, p, p]
        lib.oracle_quant_weight_nvfp4.restype = None
        lib.oracle_quant_weight_nvfp4.argtypes = [p, i64, i64, p, p, p]
        lib.oracle_pack_signs.restype = None
        lib.oracle_pack_signs.argtypes = [p, i64, i64, p]
        lib.oracle_gemm_lowrank.restype = None
        lib.oracle_gemm_lowrank.argtypes = [p, p, p, ctypes.c_float, p, p, p,
                                            i64, i64, i64, i64, p, p, p, p]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().oracle_e4m3_value(int(byte))


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def e2m1_encode(x: float, s: float) -> int:
    return int(_load().oracle_e2m1_encode(float(x), float(s)))


def e2m1_encode_n(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    xx = np.ascontiguousarray(x, dtype=np.float64).ravel()
    ss = np.ascontiguousarray(s, dtype=np.float64).ravel()
    assert xx.shape == ss.shape
    out = np.zeros(xx.shape, np.uint8)
    _load().oracle_e2m1_encode_n(_ptr(xx), _ptr(ss), xx.size, _ptr(out))
    return out


def e4m3_encode_n(v: np.ndarray) -> np.ndarray:
    vv = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.zeros(vv.shape, np.uint8)
    _load().oracle_e4m3_encode_n(_ptr(vv), vv.size, _ptr(out))
    return out


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def quant_act_fp4(x_bf16: np.ndarray):
    """x_bf16: uint16 [M][K] -> (codes uint8 [M][K/2], scales uint8 [M][K/16])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    assert K % 16 == 0
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    _load().oracle_quant_act_fp4(_ptr(x), M, K, _ptr(codes), _ptr(scales))
    return codes, scales


def quant_weight_nvfp4(w: np.ndarray):
    """w: float32 [N][K] -> (codes uint8 [N][K/2], scales uint8 [N][K/16], g float32)."""
    a = np.ascontiguousarray(w, dtype=np.float32)
    N, K = a.shape
    assert K % 16 == 0
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    g = np.zeros(1, np.float32)
    _load().oracle_quant_weight_nvfp4(_ptr(a), N, K, _ptr(codes), _ptr(scales), _ptr(g))
    return codes, scales, np.float32(g[0])


def pack_signs(signs: np.ndarray) -> np.ndarray:
    """signs: int8 [rows][cols] -> uint32 [ceil(rows/32)][cols]."""
    s = np.ascontiguousarray(signs, dtype=np.int8)
    rows, cols = s.shape
    out = np.zeros(((rows + 31) // 32, cols), np.uint32)
    _load().oracle_pack_signs(_ptr(s), rows, cols, _ptr(out))
    return out


def gemm_lowrank(x_bf16, wcode, wscale, g, V, U, alpha_bf16, parts: bool = False):
    """Method-level operands (see the C file) -> y double [M][N]
    (and, with ``parts``, the dict {y, G, C, z})."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    wc = np.ascontiguousarray(wcode, dtype=np.uint8)
    ws = np.ascontiguousarray(wscale, dtype=np.uint8)
    M, K = x.shape
    N = wc.shape[0]
    assert wc.shape == (N, K) and ws.shape == (N, K // 16)
    r = 0 if V is None else V.shape[1]
    Vc = np.ascontiguousarray(V if r else np.zeros((K, 0)), dtype=np.int8)
    Uc = np.ascontiguousarray(U if r else np.zeros((N, 0)), dtype=np.int8)
    al = np.ascontiguousarray(alpha_bf16 if r else np.zeros(0), dtype=np.uint16)
    assert Vc.shape == (K, r) and Uc.shape == (N, r) and al.shape == (r,)
    y = np.zeros((M, N), np.float64)
    G = np.zeros((M, N), np.float64) if parts else None
    C = np.zeros((M, N), np.float64) if parts else None
    z = np.zeros((M, r), np.float64) if parts else None
    _load().oracle_gemm_lowrank(_ptr(x), _ptr(wc), _ptr(ws), float(g), _ptr(Vc), _ptr(Uc),
                                _ptr(al), M, N, K, r, _ptr(y), _ptr(G), _ptr(C), _ptr(z))
    if parts:
        return {"y": y, "G": G, "C": C, "z": z}
    return y


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only; results do not
    depend on it)."""
    _load().oracle_set_num_threads(int(n))

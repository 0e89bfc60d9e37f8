"""Thin Python binding of libbiloco_hip (ctypes).

Argument marshalling only: every step runs in the library's HIP kernels.
Functions carry the C ABI's names; array arguments are torch tensors on the
GPU (device memory), passed by pointer, and calls are enqueued on torch's
current stream.  A missing library is an error: there is no other path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# another build of the same library (the host-sanitized one the tests load)
# can be named with BILOCO_HIP_LIB
LIB_PATH = os.environ.get("BILOCO_HIP_LIB") or os.path.join(_PKG, "libbiloco_hip.so")

BILOCO_OK = 0
BILOCO_ERR_INVALID_VALUE = 1
BILOCO_ERR_UNSUPPORTED = 2
BILOCO_ERR_HIP = 3
BILOCO_ERR_WORKSPACE_TOO_SMALL = 4

BILOCO_SCHED_AUTO = 0
BILOCO_SCHED_UNFUSED = 1
BILOCO_SCHED_FUSED_GEMV = 2
BILOCO_SCHED_FUSED_MFMA = 3
BILOCO_SCHED_COMPOSED = 4
BILOCO_SCHED_COMPOSED_MFMA = 5
BILOCO_SCHED_MFMA_ALLWG = 6
BILOCO_SCHED_MFMA_SIDE = 7
BILOCO_SCHED_MFMA_ZEPI = 8

EXPORTED = ["biloco_status_string", "biloco_pack_signs", "biloco_quant_act_fp4",
            "biloco_gemm_workspace_bytes", "biloco_gemm_lowrank", "biloco_gemm_lowrank_sched",
            "biloco_gemm_check", "biloco_default_schedule", "biloco_schedules_for",
            "biloco_quant_weight_nvfp4", "biloco_quant_weight_workspace_bytes",
            "biloco_peel_decompose", "biloco_peel_workspace_bytes", "biloco_gemm_lowrank_quant",
            "biloco_gemm_lowrank_quant_noalloc"]

# size of the device array biloco_gemm_lowrank_quant_noalloc works in
BILOCO_NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


class BilocoError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_name(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_weight_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64, sz, st = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                               ctypes.c_int32)
        L.biloco_status_string.restype = ctypes.c_char_p
        L.biloco_status_string.argtypes = [st]
        L.biloco_pack_signs.restype = st
        L.biloco_pack_signs.argtypes = [p, i64, i64, p, p]
        L.biloco_quant_act_fp4.restype = st
        L.biloco_quant_act_fp4.argtypes = [p, i32, i32, p, p, p]
        L.biloco_quant_weight_nvfp4.restype = st
        L.biloco_quant_weight_nvfp4.argtypes = [p, i64, i64, p, p, p, p, sz, p]
        L.biloco_quant_weight_workspace_bytes.restype = st
        L.biloco_quant_weight_workspace_bytes.argtypes = [i64, i64, ctypes.POINTER(sz)]
        L.biloco_peel_decompose.restype = st
        L.biloco_peel_decompose.argtypes = [p, i64, i64, i32, i32, p, p, p, p, p, p, p, sz, p]
        L.biloco_peel_workspace_bytes.restype = st
        L.biloco_peel_workspace_bytes.argtypes = [i64, i64, i32, ctypes.POINTER(sz)]
        L.biloco_gemm_workspace_bytes.restype = st
        L.biloco_gemm_workspace_bytes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
        gemm = [p, p, p, p, p, ctypes.c_float, p, p, p, i32, i32, i32, i32, p, p, sz]
        L.biloco_gemm_lowrank.restype = st
        L.biloco_gemm_lowrank.argtypes = gemm + [p]
        L.biloco_gemm_lowrank_sched.restype = st
        L.biloco_gemm_lowrank_sched.argtypes = gemm + [i32, p]
        L.biloco_gemm_lowrank_quant.restype = st
        L.biloco_gemm_lowrank_quant.argtypes = [p, p, p, p, p, ctypes.c_float, p, p, p, i32, i32, i32,
                                                i32, p, p, sz, i32, p]
        L.biloco_gemm_lowrank_quant_noalloc.restype = st
        L.biloco_gemm_lowrank_quant_noalloc.argtypes = [p, p, p, p, p, ctypes.c_float, p, p, p, i32,
                                                        i32, i32, i32, p, i32, p]
        L.biloco_gemm_check.restype = st
        L.biloco_gemm_check.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, i32, p, p, sz, i32]
        L.biloco_default_schedule.restype = i32
        L.biloco_default_schedule.argtypes = [i32, i32, i32, i32]
        L.biloco_schedules_for.restype = i32
        L.biloco_schedules_for.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), i32]
        _lib = L
    return _lib


def status_name(s: int) -> str:
    return lib().biloco_status_string(int(s)).decode()


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ok(status: int, what: str):
    if status != BILOCO_OK:
        raise BilocoError(status, what)


def biloco_status_string(s: int) -> str:
    return status_name(s)


def biloco_pack_signs(signs: torch.Tensor, packed: torch.Tensor | None = None, stream=None):
    """signs int8 [rows][cols] (pass V.T / U.T) -> int32 words [ceil(rows/32)][cols]."""
    rows, cols = signs.shape
    if packed is None:
        packed = torch.empty(((rows + 31) // 32, cols), dtype=torch.int32, device=signs.device)
    _ok(lib().biloco_pack_signs(_p(signs), rows, cols, _p(packed), _stream(stream)),
        "biloco_pack_signs")
    return packed


def biloco_quant_act_fp4(x_bf16: torch.Tensor, codes=None, scales=None, stream=None):
    """x bf16 [M][K] -> (codes uint8 [M][K/2], scales uint8 [M][K/16])."""
    M, K = x_bf16.shape
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x_bf16.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x_bf16.device)
    _ok(lib().biloco_quant_act_fp4(_p(x_bf16), M, K, _p(codes), _p(scales), _stream(stream)),
        "biloco_quant_act_fp4")
    return codes, scales


def biloco_quant_weight_workspace_bytes(N: int, K: int) -> int:
    out = ctypes.c_size_t(0)
    _ok(lib().biloco_quant_weight_workspace_bytes(N, K, ctypes.byref(out)),
        "biloco_quant_weight_workspace_bytes")
    return int(out.value)


def biloco_quant_weight_nvfp4(w: torch.Tensor, codes=None, scales=None, g=None, workspace=None,
                              stream=None):
    """w fp32 [N][K] -> (codes uint8 [N][K/2], scales uint8 [N][K/16], g fp32 [1]), all on w's device."""
    N, K = w.shape
    dev = w.device
    if codes is None:
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
    if g is None:
        g = torch.empty(4, dtype=torch.float32, device=dev)[:1]
    nws = biloco_quant_weight_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    _ok(lib().biloco_quant_weight_nvfp4(_p(w), N, K, _p(codes), _p(scales), _p(g), _p(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)),
        "biloco_quant_weight_nvfp4")
    return codes, scales, g


def biloco_peel_workspace_bytes(m: int, n: int, r: int) -> int:
    out = ctypes.c_size_t(0)
    _ok(lib().biloco_peel_workspace_bytes(m, n, r, ctypes.byref(out)),
        "biloco_peel_workspace_bytes")
    return int(out.value)


def biloco_peel_decompose(W: torch.Tensor, r: int, T: int, v_init: torch.Tensor,
                          want_residual: bool = True, workspace=None, stream=None):
    """W fp32 [m][n], v_init int32 words [r][ceil(n/32)] (bit set = -1) ->
    dict(u_packed [ceil(r/32)][m], v_packed [ceil(r/32)][n] (int32 words),
    alpha [r], alpha_greedy [r], R [m][n] or None), all on W's device."""
    m, n = W.shape
    dev = W.device
    RW = (r + 31) // 32
    out = {"u_packed": torch.empty((RW, m), dtype=torch.int32, device=dev),
           "v_packed": torch.empty((RW, n), dtype=torch.int32, device=dev),
           "alpha": torch.empty(r, dtype=torch.float32, device=dev),
           "alpha_greedy": torch.empty(r, dtype=torch.float32, device=dev),
           "R": torch.empty((m, n), dtype=torch.float32, device=dev) if want_residual else None}
    if workspace is None:
        workspace = torch.empty(biloco_peel_workspace_bytes(m, n, r), dtype=torch.uint8, device=dev)
    _ok(lib().biloco_peel_decompose(_p(W), m, n, r, T, _p(v_init), _p(out["u_packed"]),
                                    _p(out["v_packed"]), _p(out["alpha"]), _p(out["alpha_greedy"]),
                                    _p(out["R"]), _p(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)),
        "biloco_peel_decompose")
    return out


def biloco_gemm_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    out = ctypes.c_size_t(0)
    _ok(lib().biloco_gemm_workspace_bytes(M, N, K, r, ctypes.byref(out)),
        "biloco_gemm_workspace_bytes")
    return int(out.value)


def biloco_gemm_lowrank_sched(a_codes, a_scales, x_bf16, w_codes, w_scales, w_global_scale,
                              v_packed, u_packed, alpha_bf16, M, N, K, r, y, workspace,
                              workspace_bytes, schedule=BILOCO_SCHED_AUTO, stream=None):
    st = lib().biloco_gemm_lowrank_sched(
        _p(a_codes), _p(a_scales), _p(x_bf16), _p(w_codes), _p(w_scales), float(w_global_scale),
        _p(v_packed), _p(u_packed), _p(alpha_bf16), M, N, K, r, _p(y), _p(workspace),
        int(workspace_bytes), int(schedule), _stream(stream))
    _ok(st, "biloco_gemm_lowrank_sched")
    return y


def biloco_gemm_lowrank(a_codes, a_scales, x_bf16, w_codes, w_scales, w_global_scale, v_packed,
                        u_packed, alpha_bf16, M, N, K, r, y, workspace, workspace_bytes,
                        stream=None):
    st = lib().biloco_gemm_lowrank(
        _p(a_codes), _p(a_scales), _p(x_bf16), _p(w_codes), _p(w_scales), float(w_global_scale),
        _p(v_packed), _p(u_packed), _p(alpha_bf16), M, N, K, r, _p(y), _p(workspace),
        int(workspace_bytes), _stream(stream))
    _ok(st, "biloco_gemm_lowrank")
    return y


def biloco_gemm_lowrank_quant_noalloc(x_bf16, a_codes, a_scales, w_codes, w_scales,
                                      w_global_scale, v_packed, u_packed, alpha_bf16, M, N, K, r, y,
                                      schedule=BILOCO_SCHED_AUTO, stream=None):
    """biloco_gemm_lowrank_quant in the library's own per-GPU scratch array
    (no workspace argument; nothing is allocated)."""
    st = lib().biloco_gemm_lowrank_quant_noalloc(
        _p(x_bf16), _p(a_codes), _p(a_scales), _p(w_codes), _p(w_scales), float(w_global_scale),
        _p(v_packed), _p(u_packed), _p(alpha_bf16), M, N, K, r, _p(y), int(schedule),
        _stream(stream))
    _ok(st, "biloco_gemm_lowrank_quant_noalloc")
    return y


def biloco_gemm_lowrank_quant(x_bf16, a_codes, a_scales, w_codes, w_scales, w_global_scale,
                              v_packed, u_packed, alpha_bf16, M, N, K, r, y, workspace,
                              workspace_bytes, schedule=BILOCO_SCHED_AUTO, stream=None):
    """Quantise x into a_codes / a_scales (outputs) and compute y, in one call."""
    st = lib().biloco_gemm_lowrank_quant(
        _p(x_bf16), _p(a_codes), _p(a_scales), _p(w_codes), _p(w_scales), float(w_global_scale),
        _p(v_packed), _p(u_packed), _p(alpha_bf16), M, N, K, r, _p(y), _p(workspace),
        int(workspace_bytes), int(schedule), _stream(stream))
    _ok(st, "biloco_gemm_lowrank_quant")
    return y


def biloco_gemm_check(a_codes, a_scales, x_bf16, w_codes, w_scales, v_packed, u_packed,
                      alpha_bf16, M, N, K, r, y, workspace, workspace_bytes,
                      schedule=BILOCO_SCHED_AUTO) -> int:
    """Host-only argument check; returns the status code (no GPU needed)."""
    return int(lib().biloco_gemm_check(
        _p(a_codes), _p(a_scales), _p(x_bf16), _p(w_codes), _p(w_scales), _p(v_packed),
        _p(u_packed), _p(alpha_bf16), M, N, K, r, _p(y), _p(workspace), int(workspace_bytes),
        int(schedule)))


def biloco_default_schedule(M: int, N: int, K: int, r: int) -> int:
    return int(lib().biloco_default_schedule(M, N, K, r))


def biloco_schedules_for(M: int, N: int, K: int, r: int) -> list:
    buf = (ctypes.c_int32 * 8)()
    n = lib().biloco_schedules_for(M, N, K, r, buf, 8)
    return [int(buf[i]) for i in range(min(n, 8))]

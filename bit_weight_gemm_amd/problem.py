"""Device-resident operands of one product, built from a workloads dict.

Plumbing for tests, smoke and bench: copies the seeded host arrays to the
GPU, packs U^T / V^T and quantises x with the library's own kernels, and
owns the zero-filled workspace and the output.  No arithmetic of the method
happens here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceProblem:
    def __init__(self, d: dict, device: str = "cuda", quantize: bool = True):
        self.M, self.K, self.N, self.r = d["M"], d["K"], d["N"], d["r"]
        self.g = float(d["g"])
        self.device = device
        self.x = _dev(d["x"].view(np.int16), device)
        self.w_codes = _dev(d["wcodes_packed"], device)
        self.w_scales = _dev(d["wscales"], device)
        if self.r > 0:
            self.vT = _dev(np.ascontiguousarray(d["V"].T), device)     # [r][K] int8
            self.uT = _dev(np.ascontiguousarray(d["U"].T), device)     # [r][N] int8
            self.alpha = _dev(d["alpha"].view(np.int16), device)
            self.v_packed = B.biloco_pack_signs(self.vT)
            self.u_packed = B.biloco_pack_signs(self.uT)
        else:
            self.vT = self.uT = self.alpha = self.v_packed = self.u_packed = None
        self.ws_bytes = B.biloco_gemm_workspace_bytes(self.M, self.N, self.K, self.r)
        self.ws = torch.zeros(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.y = torch.zeros((self.M, self.N), dtype=torch.int16, device=device)
        self.a_codes = torch.empty((self.M, self.K // 2), dtype=torch.uint8, device=device)
        self.a_scales = torch.empty((self.M, self.K // 16), dtype=torch.uint8, device=device)
        if quantize:
            self.quantize()

    def quantize(self, stream=None):
        B.biloco_quant_act_fp4(self.x, self.a_codes, self.a_scales, stream=stream)

    def gemm(self, schedule: int = B.BILOCO_SCHED_AUTO, stream=None, w_codes=None,
             w_scales=None, u_packed=None, v_packed=None, y=None, ws=None):
        return B.biloco_gemm_lowrank_sched(
            self.a_codes, self.a_scales, self.x if self.r else None,
            self.w_codes if w_codes is None else w_codes,
            self.w_scales if w_scales is None else w_scales, self.g,
            self.v_packed if v_packed is None else v_packed,
            self.u_packed if u_packed is None else u_packed, self.alpha,
            self.M, self.N, self.K, self.r, self.y if y is None else y,
            self.ws if ws is None else ws, self.ws_bytes if ws is None else ws.numel(),
            schedule=schedule, stream=stream)

    def step(self, schedule: int = B.BILOCO_SCHED_AUTO, stream=None):
        """One pass of the per-call hot path: quantise x, then the product."""
        self.quantize(stream)
        return self.gemm(schedule, stream)

    def gemm_quant(self, schedule: int = B.BILOCO_SCHED_AUTO, stream=None, w_codes=None,
                   w_scales=None, u_packed=None, v_packed=None, y=None, ws=None):
        """The same pass as one call: quantise x (into a_codes / a_scales) and the
        product, the quantisation folded into the z launch where there is one."""
        return B.biloco_gemm_lowrank_quant(
            self.x, self.a_codes, self.a_scales,
            self.w_codes if w_codes is None else w_codes,
            self.w_scales if w_scales is None else w_scales, self.g,
            self.v_packed if v_packed is None else v_packed,
            self.u_packed if u_packed is None else u_packed, self.alpha,
            self.M, self.N, self.K, self.r, self.y if y is None else y,
            self.ws if ws is None else ws, self.ws_bytes if ws is None else ws.numel(),
            schedule=schedule, stream=stream)

    def y_float(self) -> np.ndarray:
        bits = self.y.cpu().numpy().view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)

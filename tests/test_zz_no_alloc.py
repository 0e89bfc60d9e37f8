"""biloco_gemm_lowrank_quant_noalloc, the entry point for callers that
cannot allocate, against biloco_gemm_lowrank_quant with a workspace of its
own: the activation codes and scales and y bit for bit (the same kernels on
the same inputs), and y against the oracle within the product's tolerance.
Calls in a row on the library's one scratch array, each smaller than the
one before, then larger again, every schedule each shape allows; a shape
whose workspace exceeds the array is refused before any HIP call."""
import numpy as np
import pytest
import torch

import oracle
from bit_weight_gemm_amd import binding as B
from bit_weight_gemm_amd import workloads as wl
from bit_weight_gemm_amd.problem import DeviceProblem
from util import check_y

pytestmark = pytest.mark.gpu


def _noalloc(p, schedule):
    c = torch.full_like(p.a_codes, 0x5A)
    s = torch.full_like(p.a_scales, 0x33)
    y = torch.zeros_like(p.y)
    B.biloco_gemm_lowrank_quant_noalloc(p.x, c, s, p.w_codes, p.w_scales, p.g, p.v_packed,
                                        p.u_packed, p.alpha, p.M, p.N, p.K, p.r, y,
                                        schedule=schedule)
    torch.cuda.synchronize()
    return c, s, y


def test_noalloc_matches_the_workspace_call():
    # shapes in the order called: large (M = 32, z over 14 K-slices), then
    # smaller ones, then the M = 1 one-launch shape, then the smallest again
    shapes = [(3, None), (2, None), (0, None), (1, None), (1, 0), (0, None)]
    for cfg, r in shapes:
        d = wl.make_config(cfg, r=r)
        assert B.biloco_gemm_workspace_bytes(d["M"], d["N"], d["K"], d["r"]) <= \
            B.BILOCO_NOALLOC_SCRATCH_BYTES
        y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                    d["alpha"])
        rc, rs = oracle.quant_act_fp4(d["x"])
        p = DeviceProblem(d, quantize=False)
        for sched in [B.BILOCO_SCHED_AUTO] + B.biloco_schedules_for(d["M"], d["N"], d["K"], d["r"]):
            print(f"config {cfg} r={d['r']} schedule {sched}", flush=True)
            p.y.zero_()
            p.gemm_quant(sched)                       # the existing entry point, own workspace
            torch.cuda.synchronize()
            c, s, y = _noalloc(p, sched)
            np.testing.assert_array_equal(c.cpu().numpy(), rc)
            np.testing.assert_array_equal(s.cpu().numpy(), rs)
            assert torch.equal(c, p.a_codes) and torch.equal(s, p.a_scales)
            assert torch.equal(y, p.y), f"config {cfg} schedule {sched}: y differs from the workspace call"
            bits = y.cpu().numpy().view(np.uint16).astype(np.uint32) << 16
            check_y(bits.view(np.float32).astype(np.float64), y_ref, f"config {cfg} schedule {sched}")


def test_noalloc_refuses_a_shape_beyond_the_array():
    M, K, N, r = 32, 16384, 16384, 1024
    assert B.biloco_gemm_workspace_bytes(M, N, K, r) > B.BILOCO_NOALLOC_SCRATCH_BYTES
    t = torch.zeros(256, dtype=torch.uint8, device="cuda")
    st = B.lib().biloco_gemm_lowrank_quant_noalloc(
        t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(), 0.01, t.data_ptr(),
        t.data_ptr(), t.data_ptr(), M, N, K, r, t.data_ptr(), 0, None)
    assert st == B.BILOCO_ERR_UNSUPPORTED

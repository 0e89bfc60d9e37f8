"""GPU parity of biloco_gemm_lowrank against the fp64 oracle.

Every schedule a shape allows is compared element by element with the
oracle on the same seeded inputs: all five decode workloads at full size,
the r = 0 plain GEMM, every M in 1..32 on a small ragged shape, partial sign
words, repeated calls on one workspace, and the captured-graph form the
benchmark times (rotated weight copies, several replays).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from bit_weight_gemm_amd import binding as B
from bit_weight_gemm_amd import workloads as wl
from bit_weight_gemm_amd.problem import DeviceProblem
from util import check_y

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def _case(cfg, r=None):
    d = wl.make_config(cfg, r=r)
    y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"])
    return d, y_ref


def _run(d, schedule, problem=None):
    p = problem or DeviceProblem(d)
    p.y.zero_()
    p.gemm(schedule)
    torch.cuda.synchronize()
    return p.y_float(), p


def _schedules(d):
    return B.biloco_schedules_for(d["M"], d["N"], d["K"], d["r"])


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_workload_all_schedules(cfg):
    d, y_ref = _case(cfg)
    p = DeviceProblem(d)
    for s in _schedules(d):
        print(f"config {cfg} schedule {s}", flush=True)
        y, _ = _run(d, s, p)
        check_y(y, y_ref, f"config {cfg} schedule {s}")


def test_config1_r0_plain_gemm():
    d, y_ref = _case(1, r=0)
    p = DeviceProblem(d)
    for s in _schedules(d):
        y, _ = _run(d, s, p)
        check_y(y, y_ref, f"r=0 schedule {s}")


@pytest.mark.parametrize("M", list(range(1, 33)))
def test_every_batch_size_ragged(M):
    K, N, r = 256, 200, 40          # N not a multiple of any tile; r has a partial word
    d = wl.make_inputs(M, K, N, r, seed=500 + M)
    y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"])
    p = DeviceProblem(d)
    for s in _schedules(d):
        y, _ = _run(d, s, p)
        check_y(y, y_ref, f"M={M} schedule {s}")


@pytest.mark.parametrize("M,K,N,r", [(1, 32, 1, 1), (2, 64, 3, 31), (4, 1024, 700, 33),
                                     (3, 2048, 64, 0), (1, 16384, 96, 96), (16, 512, 130, 512),
                                     # a K tail inside a 128-k chunk, one K-slice
                                     (17, 480, 77, 65),
                                     # several 16-row-block passes per workgroup, one K-slice
                                     (5, 256, 66000, 8),
                                     # several passes and two K-slices (batch of 32 rows)
                                     (17, 4096, 33000, 64),
                                     # many K-slices with a ragged last one
                                     (32, 13856, 40, 100),
                                     # one m-block, K of 25 .. 40 chunks in one slice of
                                     # the wide tiles: just past the narrow tiles' reach,
                                     # a K tail inside a chunk, several passes
                                     (16, 3200, 50, 1), (9, 4000, 1000, 70),
                                     (3, 5120, 70000, 33),
                                     # z over 7 and 8 K-slices of 1024: the slices'
                                     # exchange in the z launch, and in a launch of its own
                                     (20, 7168, 200, 33), (5, 8192, 300, 70),
                                     # vector schedules, activation per lane or through
                                     # LDS (64-block lanes x rows of 6, 8, 12 and 16)
                                     (2, 3072, 500, 40), (2, 4096, 500, 40),
                                     (2, 6144, 300, 33), (1, 8192, 300, 100),
                                     (1, 12288, 200, 64),
                                     # matrix cores at tiny K: scale windows reaching past
                                     # the few scale bytes of each row and of the arrays
                                     (3, 32, 17, 3), (32, 32, 40, 8), (5, 64, 16, 0),
                                     (20, 96, 33, 40)])
def test_edge_shapes(M, K, N, r):
    d = wl.make_inputs(M, K, N, r, seed=M * 1000 + N)
    y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"])
    p = DeviceProblem(d)
    for s in _schedules(d):
        y, _ = _run(d, s, p)
        check_y(y, y_ref, f"{(M, K, N, r)} schedule {s}")


def test_repeated_calls_one_workspace():
    d, y_ref = _case(0)
    p = DeviceProblem(d)
    for s in _schedules(d):
        first = None
        for it in range(200):
            p.gemm(s)
        torch.cuda.synchronize()
        y = p.y_float()
        check_y(y, y_ref, f"after 200 calls schedule {s}")
        # deterministic: one more call gives identical bits
        before = p.y.clone()
        p.gemm(s)
        torch.cuda.synchronize()
        assert torch.equal(before, p.y)


def test_two_streams_two_workspaces():
    d1, y1 = _case(0)
    d2 = wl.make_inputs(2, 512, 300, 64, seed=77)
    y2 = oracle.gemm_lowrank(d2["x"], d2["wcode"], d2["wscales"], d2["g"], d2["V"], d2["U"],
                             d2["alpha"])
    p1, p2 = DeviceProblem(d1), DeviceProblem(d2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(20):
        with torch.cuda.stream(s1):
            p1.gemm(B.BILOCO_SCHED_AUTO, stream=s1)
        with torch.cuda.stream(s2):
            p2.gemm(B.BILOCO_SCHED_AUTO, stream=s2)
    torch.cuda.synchronize()
    check_y(p1.y_float(), y1, "stream 1")
    check_y(p2.y_float(), y2, "stream 2")


_FALLBACK_SCRIPT = r"""
import os, sys
sys.path.insert(0, {root!r})
import numpy as np, torch
import oracle
from bit_weight_gemm_amd import binding as B, workloads as wl
from bit_weight_gemm_amd.problem import DeviceProblem
sys.path.insert(0, os.path.join({root!r}, 'tests'))
from util import check_y
for (M, K, N, r) in [(1, 256, 256, 16), (2, 1024, 300, 40), (1, 5120, 512, 512)]:
    d = wl.make_inputs(M, K, N, r, seed=31 + M)
    y_ref = oracle.gemm_lowrank(d['x'], d['wcode'], d['wscales'], d['g'], d['V'], d['U'], d['alpha'])
    p = DeviceProblem(d)
    for it in range(3):
        p.gemm(B.BILOCO_SCHED_FUSED_GEMV)
    torch.cuda.synchronize()
    check_y(p.y_float(), y_ref, f'fallback {{(M, K, N, r)}}')
for (M, K, N, r) in [(8, 1024, 300, 40), (32, 2048, 200, 100), (3, 512, 64, 33), (8, 1024, 200, 500),
                     (32, 4096, 300, 100), (5, 8192, 300, 70)]:
    d = wl.make_inputs(M, K, N, r, seed=41 + M)
    y_ref = oracle.gemm_lowrank(d['x'], d['wcode'], d['wscales'], d['g'], d['V'], d['U'], d['alpha'])
    p = DeviceProblem(d)
    for sched in (B.BILOCO_SCHED_MFMA_ALLWG, B.BILOCO_SCHED_MFMA_SIDE, B.BILOCO_SCHED_MFMA_ZEPI):
        if sched not in B.biloco_schedules_for(M, N, K, r):
            continue
        for it in range(3):
            p.y.zero_()
            p.gemm(sched)
        torch.cuda.synchronize()
        check_y(p.y_float(), y_ref, f'matrix-core one-launch fallback {{sched}} {{(M, K, N, r)}}')
print('FALLBACK_OK')
"""


def test_bounded_wait_fallback_forced_from_host():
    """With the wait bound forced to zero (debug knob read by the library at
    load), consumers that find z not yet published compute it themselves;
    results must still match the oracle."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, BILOCO_DEBUG_SPIN_LIMIT="0")
    out = subprocess.run([sys.executable, "-c", _FALLBACK_SCRIPT.format(root=root)], env=env,
                         capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and "FALLBACK_OK" in out.stdout, out.stdout + out.stderr


def _fused_quant_case(d, y_ref, schedules):
    p = DeviceProblem(d, quantize=False)
    rc, rs = oracle.quant_act_fp4(d["x"])
    for s in schedules:
        p.a_codes.fill_(0x5A)
        p.a_scales.fill_(0x33)
        p.y.zero_()
        p.gemm_quant(s)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(p.a_codes.cpu().numpy(), rc, err_msg=f"schedule {s}")
        np.testing.assert_array_equal(p.a_scales.cpu().numpy(), rs, err_msg=f"schedule {s}")
        check_y(p.y_float(), y_ref, f"quantise + product, schedule {s}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_quant_and_product_in_one_call(cfg):
    # biloco_gemm_lowrank_quant: the activation codes and scales it writes are
    # the oracle's bit for bit, and y is within tolerance, on every schedule
    d, y_ref = _case(cfg)
    _fused_quant_case(d, y_ref, [B.BILOCO_SCHED_AUTO] + _schedules(d))


@pytest.mark.parametrize("M,K,N,r", [(2, 1024, 300, 40), (17, 480, 77, 65), (5, 256, 200, 0)])
def test_quant_and_product_in_one_call_edges(M, K, N, r):
    d = wl.make_inputs(M, K, N, r, seed=900 + M)
    y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"])
    _fused_quant_case(d, y_ref, [B.BILOCO_SCHED_AUTO] + _schedules(d))


# The quantising vector-schedule calls quantise x while each wave's first
# row streams in: every activation layout they take (per-lane blocks or the
# workgroup's LDS copy, 1 to 16 blocks per lane), with and without z, with
# rows per wave from 1 to the register budget's maximum.
@pytest.mark.parametrize("M,K", [(1, 256), (1, 1056), (1, 5120), (1, 16384), (2, 256), (2, 3072),
                                 (2, 8192)])
@pytest.mark.parametrize("N,r", [(77, 0), (2300, 0), (77, 9), (2300, 512)])
def test_quant_vector_schedule_layouts(M, K, N, r):
    d = wl.make_inputs(M, K, N, r, seed=1300 + M + K + N + r)
    y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"])
    scheds = [B.BILOCO_SCHED_AUTO] + [s for s in _schedules(d)
                                      if s in (B.BILOCO_SCHED_UNFUSED, B.BILOCO_SCHED_FUSED_GEMV)]
    _fused_quant_case(d, y_ref, scheds)


def _degenerate(d, what):
    """Degenerate operands of the method: the oracle's y for them has a plain
    form, checked before the GPU is compared with it."""
    d = dict(d)
    if what == "x_zero":
        d["x"] = np.zeros_like(d["x"])                       # y = 0 exactly
    elif what == "r_codes_zero":
        d["wcode"] = np.zeros_like(d["wcode"])               # y = correction only
        d["wcodes_packed"] = wl.pack_nibbles(d["wcode"])
    elif what == "alpha_zero":
        d["alpha"] = np.zeros_like(d["alpha"])               # y = FP4 product only
    elif what == "signs_plus":
        d["U"] = np.ones_like(d["U"])                        # C = (sum alpha)(sum_k x)
        d["V"] = np.ones_like(d["V"])
    elif what == "negative_zero_codes":
        d["wcode"] = np.where(d["wcode"] == 0, 8, d["wcode"]).astype(np.uint8)   # -0 codes
        d["wcodes_packed"] = wl.pack_nibbles(d["wcode"])
    return d


@pytest.mark.parametrize("what", ["x_zero", "r_codes_zero", "alpha_zero", "signs_plus",
                                  "negative_zero_codes"])
@pytest.mark.parametrize("M", [1, 2, 8, 32])
def test_degenerate_operands(what, M):
    base = wl.make_inputs(M, 1024, 520, 96, seed=70 + M)
    d = _degenerate(base, what)
    y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"])
    parts = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"], parts=True)
    if what == "x_zero":
        assert not np.any(y_ref)
    elif what == "r_codes_zero":
        assert not np.any(parts["G"])
    elif what == "alpha_zero":
        assert not np.any(parts["C"])
    elif what == "signs_plus":
        xs = wl.bf16_bits_to_f32(d["x"]).astype(np.float64).sum(axis=1)
        al = wl.bf16_bits_to_f32(d["alpha"]).astype(np.float64).sum()
        np.testing.assert_allclose(parts["C"], np.outer(xs * al, np.ones(d["N"])), rtol=1e-12,
                                   atol=1e-12)
    p = DeviceProblem(d)
    for s in _schedules(d):
        y, _ = _run(d, s, p)
        if what == "x_zero":
            assert not np.any(y), f"schedule {s}: y not exactly zero"
        else:
            check_y(y, y_ref, f"{what} M={M} schedule {s}")


@pytest.mark.parametrize("M,r", [(1, 1500), (3, 1500), (32, 2048)])
def test_rank_above_1024(M, r):
    # ranks the pages do not reach: the schedules that take them must stay exact
    d = wl.make_inputs(M, 512, 300, r, seed=5 + r)
    y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"])
    p = DeviceProblem(d)
    scheds = _schedules(d)
    assert scheds, "no schedule takes this shape"
    for s in scheds:
        y, _ = _run(d, s, p)
        check_y(y, y_ref, f"M={M} r={r} schedule {s}")


@pytest.mark.parametrize("cfg,sched", [(1, B.BILOCO_SCHED_AUTO), (2, B.BILOCO_SCHED_AUTO),
                                      (3, B.BILOCO_SCHED_AUTO), (4, B.BILOCO_SCHED_AUTO),
                                      (1, B.BILOCO_SCHED_FUSED_GEMV), (1, B.BILOCO_SCHED_FUSED_MFMA),
                                      (2, B.BILOCO_SCHED_MFMA_ALLWG), (3, B.BILOCO_SCHED_MFMA_ALLWG),
                                      (4, B.BILOCO_SCHED_MFMA_ALLWG)])
def test_graph_replay_as_timed(cfg, sched):
    """The form the benchmark times: quantise-and-multiply calls captured once
    in a graph over rotated copies of the weights, replayed several times with
    eager work in between.  Every call of every replay gives the eager call's
    bits (the eager call itself is checked against the oracle), and the
    activation codes and scales it writes are the oracle's."""
    d, y_ref = _case(cfg)
    p = DeviceProblem(d, quantize=False)
    rc, rs = oracle.quant_act_fp4(d["x"])
    p.gemm_quant(sched)
    torch.cuda.synchronize()
    check_y(p.y_float(), y_ref, f"config {cfg} schedule {sched} eager")
    y_eager = p.y.clone()
    n_sets, calls = 3, 6
    wc = [p.w_codes.clone() for _ in range(n_sets)]
    ws = [p.w_scales.clone() for _ in range(n_sets)]
    up = [p.u_packed.clone() for _ in range(n_sets)] if p.r else [None] * n_sets
    vp = [p.v_packed.clone() for _ in range(n_sets)] if p.r else [None] * n_sets
    ys = [torch.empty_like(p.y) for _ in range(calls)]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for i in range(calls):
            k = i % n_sets
            p.gemm_quant(sched, stream=st, w_codes=wc[k], w_scales=ws[k], u_packed=up[k],
                         v_packed=vp[k], y=ys[i])
    torch.cuda.synchronize()
    for rep in range(3):
        for t in ys:
            t.fill_(0x3F00 + rep)
        p.a_codes.fill_(0x5A)
        p.a_scales.fill_(0x33)
        torch.cuda.synchronize()
        print(f"config {cfg} schedule {sched} replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(ys):
            assert torch.equal(t, y_eager), f"config {cfg} schedule {sched} replay {rep} call {i}"
        np.testing.assert_array_equal(p.a_codes.cpu().numpy(), rc, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(p.a_scales.cpu().numpy(), rs, err_msg=f"replay {rep}")


# The one-launch vector schedule applies z through sign tables of 4 ranks,
# 64 groups per lane round: ranks on either side of every group, word and
# round boundary, at both batch sizes it takes.
@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("r", [1, 3, 4, 5, 31, 32, 33, 255, 256, 257, 511, 513, 1023, 1024])
def test_vector_schedule_rank_boundaries(M, r):
    K, N = 640, 300
    d = wl.make_inputs(M, K, N, r, seed=900 + 7 * r + M)
    y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"])
    assert B.BILOCO_SCHED_FUSED_GEMV in _schedules(d)
    p = DeviceProblem(d)
    for rep in range(2):          # the second call finds the first call's tags in the workspace
        y, _ = _run(d, B.BILOCO_SCHED_FUSED_GEMV, p)
        check_y(y, y_ref, f"M={M} r={r} call {rep}")

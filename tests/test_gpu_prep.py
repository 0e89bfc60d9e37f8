"""GPU parity of the operand-preparation kernels: bit-exact against the oracle.

biloco_pack_signs (sign words) and biloco_quant_act_fp4 (FP4 codes and E4M3
scales) are integer/byte results: every word and byte must match.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from bit_weight_gemm_amd import binding as B
from bit_weight_gemm_amd import workloads as wl
from bit_weight_gemm_amd.problem import DeviceProblem
from util import check_y

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gpu_pack(signs: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(signs)).cuda()
    out = B.biloco_pack_signs(t)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def _gpu_quant(x_bits: np.ndarray):
    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()
    c, s = B.biloco_quant_act_fp4(t)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("rows,cols", [(16, 256), (512, 5120), (512, 13824), (1024, 8192),
                                       (40, 33), (1, 1), (95, 300), (33, 4097)])
def test_pack_bit_exact(rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    s = rng.integers(-3, 3, (rows, cols), dtype=np.int8)
    np.testing.assert_array_equal(_gpu_pack(s), oracle.pack_signs(s))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_pack_workload_factors(cfg):
    d = wl.make_config(cfg)
    for F in (d["V"], d["U"]):
        FT = np.ascontiguousarray(F.T)
        np.testing.assert_array_equal(_gpu_pack(FT), oracle.pack_signs(FT))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_quant_bit_exact_workloads(cfg):
    d = wl.make_config(cfg)
    c, s = _gpu_quant(d["x"])
    rc, rs = oracle.quant_act_fp4(d["x"])
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def test_quant_golden_blocks():
    rows, scales, codes = [], [], []
    with open(os.path.join(GOLDEN, "quant_act_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if line.startswith("x "):
                rows.append([float(t) for t in line.split()[1:]])
            elif line.startswith("scale "):
                scales.append(int(line.split()[1], 16))
            elif line.startswith("codes "):
                codes.append([int(t, 16) for t in line.split()[1:]])
    # place the 16-element blocks side by side in one row of K = 16 * n (padded to K % 32 == 0)
    n = len(rows)
    K = 32 * ((16 * n + 31) // 32)
    x = np.zeros((1, K), np.float32)
    for i, r in enumerate(rows):
        x[0, 16 * i:16 * i + 16] = r
    c, s = _gpu_quant(wl.to_bf16_bits(x))
    for i in range(n):
        assert s[0, i] == scales[i], (i, hex(s[0, i]))
        assert list(c[0, 8 * i:8 * i + 8]) == codes[i], (i, [hex(v) for v in c[0, 8 * i:8 * i + 8]])


def test_quant_every_bf16_amax():
    # one block per positive finite bf16 amax; the other 15 entries are fixed
    # fractions of it (exercising many code decisions, ties included)
    amax_bits = np.arange(1, 0x7F80, dtype=np.uint32)
    nblk = amax_bits.size
    amax = (amax_bits << 16).view(np.float32)
    frac = np.array([1, -1, .5, -.25, .75, .125, -.625, .375, 0, -0.0, .9, -.05, .3125, .8125,
                     -.4375, .0625], np.float32)
    blocks = amax[:, None] * frac[None, :]
    pad = (-nblk) % 512
    blocks = np.concatenate([blocks, np.zeros((pad, 16), np.float32)])
    x = wl.to_bf16_bits(blocks.reshape(-1, 512 * 16))
    c, s = _gpu_quant(x)
    rc, rs = oracle.quant_act_fp4(x)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def test_quant_random_binades_and_zeros():
    rng = np.random.default_rng(99)
    f = rng.standard_normal((32, 4096)).astype(np.float32)
    f *= (2.0 ** rng.integers(-30, 30, (32, 256)).astype(np.float32)).repeat(16, axis=1)
    f[3, :64] = 0.0
    f[4, 16:48] = -0.0
    f[5, ::3] = 0.0
    x = wl.to_bf16_bits(f)
    c, s = _gpu_quant(x)
    rc, rs = oracle.quant_act_fp4(x)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


# ---------------------------------------------------------------- NVFP4 weights
def _gpu_wquant(w: np.ndarray):
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).cuda()
    c, s, g = B.biloco_quant_weight_nvfp4(t)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), np.float32(g.cpu().numpy()[0])


def _check_wquant(w: np.ndarray):
    c, s, g = _gpu_wquant(w)
    rc, rs, rg = oracle.quant_weight_nvfp4(w)
    assert g.tobytes() == rg.tobytes(), (g, rg)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


# (N, K): the decode shapes' R, a ragged tail tile of both passes, a single
# block, fewer float4 than one wave, and a shape where every workgroup of
# both passes loops over several tiles
@pytest.mark.parametrize("N,K,outliers", [(5120, 5120, False), (13824, 5120, True),
                                          (5120, 13824, False), (33, 528, False), (1, 16, False),
                                          (3, 48, True), (8192, 1040, True)])
def test_wquant_bit_exact(N, K, outliers):
    _check_wquant(wl.make_residual(N, K, seed=N + K, outliers=outliers))


def test_wquant_golden_rows():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "quant_weight_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            if key == "case":
                cur = {}
                cases.append(cur)
            else:
                cur[key] = rest.split()
    for case in cases:
        w = np.array([[float(t) for t in case["w"]]], np.float32)
        c, s, g = _gpu_wquant(w)
        assert float(g) == float(case["g"][0])
        assert s[0].tolist() == [int(t, 16) for t in case["scales"]]
        assert c[0].tolist() == [int(t, 16) for t in case["codes"]]


def test_wquant_zero_and_tiny_magnitudes():
    w = np.zeros((16, 256), np.float32)
    w[2, 7] = -0.0
    _check_wquant(w)                                  # g = 1, zero scales, signed zeros
    rng = np.random.default_rng(5)
    # g either side of the fast path's limit 2^-90, g normal but tiny, g
    # subnormal, subnormal inputs, and magnitudes near the top of fp32
    for scale in (1e-22, 5e-25, 1e-30, 1e-36, 1e-40, 1e37):
        _check_wquant((scale * rng.standard_normal((64, 512))).astype(np.float32))


def test_wquant_every_block_scale_and_ties():
    # one row per positive E4M3 scale byte: its block maximum is 6 * scale * g
    # with g fixed by a first block of amax 2688, and the other entries are
    # multiples of d on the E2M1 midpoints (exact ties) and just beside them
    sv = torch.arange(1, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    rows = []
    for d in sv:
        blk = np.zeros(32, np.float32)
        blk[0] = 2688.0
        b = blk[16:]
        b[0] = 6.0 * d
        b[1:8] = mids * d
        b[8:15] = -np.nextafter(mids * d, np.float32(np.inf))
        b[15] = np.nextafter(mids[3] * d, np.float32(0))
        rows.append(blk)
    _check_wquant(np.stack(rows))


@pytest.mark.parametrize("shape", [("cfg", 0), ("cfg", 1), (8, 5120, 1536, 512),
                                   (32, 13824, 640, 512), (32, 8192, 1024, 1024)],
                         ids=["config0", "config1", "M8", "M32-K13824", "M32-r1024"])
def test_wquant_feeds_gemm(shape):
    # the quantiser's output (with its small and saturated block scales and
    # outlier columns) is the product's residual operand, on every schedule:
    # the vector schedules at M = 1 and the matrix cores at M = 8 and 32
    if shape[0] == "cfg":
        d = wl.make_config(shape[1])
        seed = 11 + shape[1]
    else:
        M, K, N, r = shape
        d = wl.make_inputs(M, K, N, r, seed=K + N)
        seed = M + K
    w = wl.make_residual(d["N"], d["K"], seed=seed, outliers=True)
    c, s, g = _gpu_wquant(w)
    d["wcodes_packed"], d["wscales"], d["g"] = c, s, g
    d["wcode"] = np.stack([c & 15, c >> 4], axis=-1).reshape(d["N"], d["K"])
    y_ref = oracle.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"],
                                d["alpha"])
    p = DeviceProblem(d)
    for sched in B.biloco_schedules_for(d["M"], d["N"], d["K"], d["r"]):
        p.y.zero_()
        p.gemm(sched)
        torch.cuda.synchronize()
        check_y(p.y_float(), y_ref, f"{shape} schedule {sched} with quantised R")

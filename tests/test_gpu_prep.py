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

"""Pins of the oracle's activation quantiser and sign packer.

* quant: hand-derived blocks (golden file), the scale byte against torch's
  E4M3 cast of float32(amax/6) over every bf16 amax, and the nearest-even
  property of every code on random and outlier-heavy rows.
* pack: numpy's packbits (little bit order) as an independent packer,
  popcounts, partial last words, and the storage identity of the BiLoCo
  README's intro (binary rank 512 costs what bf16 rank 32 costs).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from bit_weight_gemm_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _blocks():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "quant_act_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            if key == "case":
                cur = {"name": rest}
                cases.append(cur)
            elif key == "x":
                cur["x"] = [float(t) for t in rest.split()]
            elif key == "scale":
                cur["scale"] = int(rest, 16)
            elif key == "codes":
                cur["codes"] = [int(t, 16) for t in rest.split()]
    return cases


@pytest.mark.parametrize("case", _blocks(), ids=lambda c: c["name"])
def test_quant_golden_blocks(case):
    xf = np.array(case["x"], np.float32)
    xb = wl.to_bf16_bits(xf)
    # the fixture values are exact in bf16
    assert np.array_equal(wl.bf16_bits_to_f32(xb), xf)
    codes, scales = oracle.quant_act_fp4(xb.reshape(1, 16))
    assert scales[0, 0] == case["scale"], hex(scales[0, 0])
    assert list(codes[0]) == case["codes"], [hex(c) for c in codes[0]]


def test_quant_scale_matches_torch_for_every_bf16_amax():
    # one block per amax value: x = [amax, 0, ...]; scale = E4M3(fp32(amax/6))
    bits = np.arange(0, 0x4520, dtype=np.uint32)   # bf16 values up to ~2560 (amax/6 < 448)
    amax = (bits << 16).view(np.float32)
    x = np.zeros((bits.size, 16), np.uint16)
    x[:, 0] = bits.astype(np.uint16)
    # rows of 16: M = count, K = 16
    _, scales = oracle.quant_act_fp4(x)
    ref = torch.from_numpy(amax / np.float32(6.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(scales[:, 0] != ref)[0]
    assert bad.size == 0, [(float(amax[i]), hex(scales[i, 0]), hex(ref[i])) for i in bad[:8]]


def _check_nearest_even(x_bits, codes, scales):
    M, K = x_bits.shape
    e2 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)
    x = wl.bf16_bits_to_f32(x_bits).astype(np.float64)
    c = np.empty((M, K), np.uint8)
    c[:, 0::2] = codes & 15
    c[:, 1::2] = codes >> 4
    s = np.array([oracle.e4m3_value(b) for b in range(256)])[scales]      # [M][K/16]
    s_full = np.repeat(s, 16, axis=1)
    # sign bit = sign of x
    assert np.array_equal((c >> 3).astype(bool), np.signbit(x))
    nz = s_full > 0
    t = np.where(nz, np.abs(x) / np.where(nz, s_full, 1.0), 0.0)
    t = np.minimum(t, 6.0)
    d = np.abs(e2[None, None, :] - t[:, :, None])
    dmin = d.min(axis=2)
    chosen = d[np.arange(M)[:, None], np.arange(K)[None, :], c & 7]
    assert np.all(chosen == dmin)
    ties = (d == dmin[:, :, None]).sum(axis=2) > 1
    assert np.all(((c & 7) % 2 == 0) | ~ties)
    # amax rule: scale is E4M3 of amax/6
    amax = np.abs(x).reshape(M, K // 16, 16).max(axis=2)
    ref = torch.from_numpy((amax / 6.0).astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(ref.view(torch.uint8).numpy(), scales)


@pytest.mark.parametrize("cfg", [0, 2])
def test_quant_nearest_even_on_workload_rows(cfg):
    d = wl.make_config(cfg)
    x = d["x"][:, :4096] if d["x"].shape[1] > 4096 else d["x"]
    codes, scales = oracle.quant_act_fp4(x)
    _check_nearest_even(x, codes, scales)


def test_quant_nearest_even_random_scales_of_magnitude():
    rng = np.random.default_rng(123)
    # rows spanning many binades, exact zeros, negative zeros and ties
    f = rng.standard_normal((6, 512)).astype(np.float32) * (10.0 ** rng.integers(-6, 4, (6, 1)))
    f[0, :16] = 0.0
    f[1, 16:32] = -0.0
    f[2, 32:48] = np.array([6, 3, 1.5, .75, .25, 5, 2.5, 1.25, 3.5, 1.75, 0, 0, 0, 0, 0, 0], np.float32)
    x = wl.to_bf16_bits(f)
    codes, scales = oracle.quant_act_fp4(x)
    _check_nearest_even(x, codes, scales)


# ----------------------------------------------------------------- packing

def _packbits_route(signs):
    """Independent packer: numpy packbits with little bit order along the rank axis."""
    rows, cols = signs.shape
    W = (rows + 31) // 32
    bits = np.zeros((W * 32, cols), np.uint8)
    bits[:rows] = (signs < 0)
    b = np.packbits(bits.T, axis=1, bitorder="little")      # [cols][W*4] bytes
    return np.ascontiguousarray(b).view("<u4").T.copy()      # [W][cols]


@pytest.mark.parametrize("rows,cols", [(16, 256), (32, 7), (40, 33), (512, 300), (1, 5), (95, 64)])
def test_pack_vs_packbits(rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    s = (1 - 2 * rng.integers(0, 2, (rows, cols))).astype(np.int8)
    got = oracle.pack_signs(s)
    assert got.shape == ((rows + 31) // 32, cols)
    assert np.array_equal(got, _packbits_route(s))
    # popcount of every word = number of -1 entries in its 32-row group
    pc = np.array([[bin(int(w)).count("1") for w in row] for row in got])
    neg = np.zeros_like(pc)
    for w in range(got.shape[0]):
        neg[w] = (s[32 * w:32 * w + 32] < 0).sum(axis=0)
    assert np.array_equal(pc, neg)
    # bits past the last row are zero
    if rows % 32:
        assert np.all(got[-1] >> np.uint32(rows % 32) == 0)


def test_pack_bit_positions():
    s = np.ones((64, 3), np.int8)
    s[0, 0] = -1       # word 0, bit 0 of column 0
    s[31, 1] = -1      # word 0, bit 31 of column 1
    s[33, 2] = -1      # word 1, bit 1 of column 2
    got = oracle.pack_signs(s)
    assert got.tolist() == [[1, 1 << 31, 0], [0, 0, 2]]


def test_pack_zero_counts_as_plus():
    s = np.zeros((32, 2), np.int8)
    s[5, 1] = -3
    assert oracle.pack_signs(s).tolist() == [[0, 1 << 5]]


def test_storage_identity_rank512_equals_bf16_rank32():
    # BiLoCo intro: a binary rank-one term is 16x cheaper than a bf16 one, so
    # bf16 rank 32 buys binary rank 512.  Packed U and V for N=K=5120, r=512:
    N = K = 5120
    r = 512
    packed_bytes = 4 * ((r + 31) // 32) * (N + K)
    bf16_rank32_bytes = 2 * 32 * (N + K)
    assert packed_bytes == bf16_rank32_bytes
    sV = np.ones((r, 64), np.int8)
    assert oracle.pack_signs(sV).nbytes == r // 8 * 64

"""Evidence for the matrix-core operand form (BiLoCo README, section "Kernel":
the FP4 product with per-16 E4M3 block scales).

Dequantising an E2M1 code times its E4M3 block scale into f16 or bf16 is
exact: every such product has at most 6 significant bits.  Folding the block
scale into an fp8 (E4M3) operand instead rounds those products to 4
significant bits.  At the decode shape M = 1, K = N = 5120, r = 512 that
rounding alone puts a large share of the outputs outside the parity bound
|err| <= 8e-3 |y| + 1e-3 rms(y), so the fold is rejected by measurement.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_weight_gemm_amd import workloads as wl

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                 -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _e4m3_bytes_to_f64(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _round_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _significant_bits(v: float) -> int:
    if v == 0.0:
        return 0
    m, _ = np.frexp(abs(v))          # v = m 2^e, 0.5 <= m < 1
    bits = 0
    while m != 0.0:
        m = m * 2.0
        m -= np.floor(m)
        bits += 1
    return bits


def test_code_times_scale_is_exact_in_f16_and_bf16():
    finite = [b for b in range(256) if np.isfinite(_e4m3_bytes_to_f64(np.array([b]))[0])]
    scales = _e4m3_bytes_to_f64(np.array(finite, dtype=np.uint8))
    worst = 0
    for s in scales:
        for c in E2M1:
            p = float(c) * float(s)
            worst = max(worst, _significant_bits(p))
            if p != 0.0:
                assert np.float64(np.float16(p)) == p          # f16 holds it exactly
                assert float(torch.tensor(p, dtype=torch.float64).to(torch.bfloat16).double()) == p
    assert worst == 6


def test_fp8_folded_scales_miss_the_parity_bound():
    d = wl.make_config(1)
    M, K = d["M"], d["K"]
    parts = O.gemm_lowrank(d["x"], d["wcode"], d["wscales"], d["g"], d["V"], d["U"], d["alpha"],
                           parts=True)
    codes, scales = O.quant_act_fp4(d["x"])
    a_codes = np.empty((M, K), np.uint8)
    a_codes[:, 0::2] = codes & 15
    a_codes[:, 1::2] = codes >> 4
    xa = E2M1[a_codes] * np.repeat(_e4m3_bytes_to_f64(scales), 16, axis=1)
    wr = E2M1[d["wcode"]] * np.repeat(_e4m3_bytes_to_f64(d["wscales"]), 16, axis=1)
    g = float(d["g"])
    exact = (xa @ wr.T) * g
    # the exact operands reproduce the oracle's product term
    assert np.array_equal(exact, parts["G"])
    # fold: each operand rounded to E4M3 (a power-of-two pre-scale keeps the
    # values under E4M3's maximum and changes no rounding)
    sh = 2.0 ** -3
    folded = (_round_e4m3(xa * sh) / sh) @ (_round_e4m3(wr * sh) / sh).T * g
    y = parts["y"]
    bound = 8e-3 * np.abs(y) + 1e-3 * np.sqrt(np.mean(y ** 2))
    over = np.mean(np.abs(folded - exact) > bound)
    print(f"outputs over the bound: {over:.4f}, worst err/bound {np.max(np.abs(folded - exact) / bound):.2f}")
    assert over > 0.05

"""Pins of the oracle's NVFP4 weight quantiser (the residual R).

* hand-derived rows (golden file: exact ties, saturation at 448, a subnormal
  scale, an all-zero matrix);
* the global scale against numpy's float32 division;
* every block scale against torch's E4M3 cast of the float32 quotient chain;
* every code: the nearest of the eight E2M1 magnitudes to the float32
  quotient, ties to the even code, found by brute force in fp64;
* the reconstruction g * scale * e2m1(code) within half the local grid step
  of every non-saturated weight, on random and outlier-heavy matrices.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "quant_weight_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            if key == "case":
                cur = {"name": rest}
                cases.append(cur)
            elif key == "w":
                cur["w"] = [float(t) for t in rest.split()]
            elif key == "g":
                cur["g"] = float(rest)
            elif key == "scales":
                cur["scales"] = [int(t, 16) for t in rest.split()]
            elif key == "codes":
                cur["codes"] = [int(t, 16) for t in rest.split()]
    return cases


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_rows(case):
    w = np.array([case["w"]], np.float32)
    codes, scales, g = oracle.quant_weight_nvfp4(w)
    assert float(g) == case["g"]
    assert scales[0].tolist() == case["scales"]
    assert codes[0].tolist() == case["codes"]


def _decode(codes):
    lo, hi = codes & 15, codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    mag = E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag), c


def _matrices():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((48, 512)).astype(np.float32)
    b = a.copy()
    b[:, rng.choice(512, 5, replace=False)] *= 40.0      # outlier columns
    c = (rng.standard_normal((16, 256)) * 1e-3).astype(np.float32)
    c[3, 17] = 7.5                                        # one dominant weight
    return {"normal": a, "outliers": b, "one_peak": c}


@pytest.mark.parametrize("name", ["normal", "outliers", "one_peak"])
def test_scales_codes_against_independent_routes(name):
    w = _matrices()[name]
    codes, scales, g = oracle.quant_weight_nvfp4(w)
    # global scale: numpy float32 division
    amax = np.float32(np.abs(w).max())
    assert g == np.float32(amax / np.float32(2688.0))
    # block scales: torch's E4M3 cast of fp32(fp32(a/6)/g), below the saturation point
    N, K = w.shape
    a = np.abs(w).reshape(N, K // 16, 16).max(axis=2).astype(np.float32)
    q = (a / np.float32(6.0)).astype(np.float32) / g
    q = q.astype(np.float32)
    ok = q < 448.0
    ref = torch.from_numpy(q[ok].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales[ok], ref)
    assert np.all(scales[~ok] == 0x7E)
    # codes: brute force nearest magnitude to the float32 quotient, ties to even code
    sval = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    d = (np.repeat(sval, 16, axis=1) * g).astype(np.float32)
    tq = np.where(d > 0, (np.abs(w) / np.where(d > 0, d, 1)).astype(np.float32), 0).astype(np.float64)
    tq = np.minimum(tq, 6.0)
    dist = np.abs(E2M1_MAG[None, None, :] - tq[:, :, None])
    best = dist.min(axis=2, keepdims=True)
    cand = dist == best
    # among the nearest, the even code (ties): the smallest even index present
    idx = np.where(cand & (np.arange(8) % 2 == 0)[None, None, :], np.arange(8), 99).min(axis=2)
    idx = np.where(idx == 99, dist.argmin(axis=2), idx)
    _, c = _decode(codes)
    assert np.array_equal(c & 7, idx)
    assert np.array_equal((c & 8) != 0, np.signbit(w))
    # reconstruction within half the local grid step (non-saturated weights)
    val, _ = _decode(codes)
    rec = val * d.astype(np.float64)
    step = np.where(np.abs(w) / np.maximum(d, 1e-30) < 2.0, 0.5, np.where(np.abs(w) / np.maximum(d, 1e-30) < 4.0, 1.0, 2.0))
    sat = np.abs(w) > 6.0 * d
    err = np.abs(rec - w.astype(np.float64))
    assert np.all(err[~sat] <= 0.5 * step[~sat] * d[~sat] * (1 + 1e-6) + 1e-30)


def test_all_zero_matrix():
    w = np.zeros((3, 64), np.float32)
    w[1, 5] = -0.0
    codes, scales, g = oracle.quant_weight_nvfp4(w)
    assert g == 1.0
    assert not scales.any()
    _, c = _decode(codes)
    assert np.array_equal(c, np.where(np.signbit(w), 8, 0))

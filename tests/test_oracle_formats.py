"""Pins of the oracle's element formats against routes that do not share its code.

* E2M1 decode: the 16-entry table of the format definition (golden file).
* E4M3 decode / encode: torch's float8_e4m3fn casts (round to nearest even).
* E2M1 encode: exhaustive sweep of every positive finite bf16 value against
  every positive finite E4M3 scale, checked by the threshold formulation of
  nearest-even rounding and by the optimality property of the result.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    assert sorted(vals) == list(range(16))
    return vals


def test_e2m1_decode_table():
    g = _e2m1_golden()
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert v == g[c], (c, v, g[c])
        # the sign of zero is part of the code
        assert np.signbit(v) == np.signbit(g[c]) or v != 0.0


def test_e4m3_decode_all_bytes_vs_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    for byte in range(256):
        v = oracle.e4m3_value(byte)
        if np.isnan(ref[byte]):
            assert np.isnan(v), byte
        else:
            assert v == ref[byte], (hex(byte), v, ref[byte])
    # spot facts of the format
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6


def _torch_e4m3(v):
    t = torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_encode_vs_torch_bf16_grid():
    # every non-negative finite bf16 value below 448, plus exact midpoints of
    # neighbouring E4M3 values and their float32 neighbours
    bits = np.arange(0, 0x43E0, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    e4 = np.array([oracle.e4m3_value(b) for b in range(0x7F)], np.float64)
    mids = ((e4[1:] + e4[:-1]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    allv = np.concatenate([vals, mids, near, e4.astype(np.float32)]).astype(np.float32)
    got = oracle.e4m3_encode_n(allv.astype(np.float64))
    ref = _torch_e4m3(allv)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(allv[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_encode_saturates():
    for v in [448.0, 450.0, 463.9, 464.0, 479.0, 480.0, 1e6, float(np.finfo(np.float32).max)]:
        assert oracle.e4m3_encode(v) == 0x7E
    assert oracle.e4m3_encode(0.0) == 0x00
    # ties to even mantissa at 1.0625 (between 1.0 and 1.125) and at 2^-10
    assert oracle.e4m3_encode(1.0625) == 0x38
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00
    assert oracle.e4m3_encode(1.5 * 2.0 ** -9) == 0x02


def _e2m1_by_thresholds(t):
    """Nearest-even E2M1 magnitude code by comparing with the midpoints."""
    t = np.asarray(t, np.float64)
    c = np.full(t.shape, 7, np.uint8)
    c[t <= 5.0] = 6
    c[t < 3.5] = 5
    c[t <= 2.5] = 4
    c[t < 1.75] = 3
    c[t <= 1.25] = 2
    c[t < 0.75] = 1
    c[t <= 0.25] = 0
    return c


def test_e2m1_encode_exhaustive_bf16_by_e4m3():
    g = _e2m1_golden()
    mags = np.array([g[c] for c in range(8)])
    xb = np.arange(1, 0x7F80, dtype=np.uint32)               # positive finite bf16
    x = (xb << 16).view(np.float32).astype(np.float64)
    sb = np.array([b for b in range(1, 0x7F)], np.uint32)    # positive finite E4M3
    s = np.array([oracle.e4m3_value(b) for b in sb], np.float64)
    total = 0
    for sign in (1.0, -1.0):
        for j in range(0, s.size, 18):
            ss = np.repeat(s[j:j + 18], x.size)
            xx = np.tile(sign * x, min(18, s.size - j))
            got = oracle.e2m1_encode_n(xx, ss)
            t = np.abs(xx) / ss
            ref = _e2m1_by_thresholds(t) | (np.uint8(8) if sign < 0 else np.uint8(0))
            assert np.array_equal(got, ref), (j, np.nonzero(got != ref)[0][:5])
            # optimality: no magnitude is strictly nearer than the chosen one
            d = np.abs(mags[got & 7] - np.minimum(t, 1e30))
            assert np.all(d <= np.min(np.abs(mags[None, :] - t[:, None]), axis=1) + 0.0)
            total += got.size
    assert total == 2 * 32639 * 126


def test_e2m1_encode_special():
    assert oracle.e2m1_encode(-0.0, 1.0) == 8
    assert oracle.e2m1_encode(0.0, 1.0) == 0
    assert oracle.e2m1_encode(5.0, 0.0) == 0
    assert oracle.e2m1_encode(-5.0, 0.0) == 8
    assert oracle.e2m1_encode(100.0, 1.0) == 7
    assert oracle.e2m1_encode(-0.2, 1.0) == 8


def test_bf16_value_all_finite():
    b = np.arange(65536, dtype=np.uint32)
    ref = (b << 16).view(np.float32)
    idx = np.nonzero(np.isfinite(ref))[0][::7]
    for i in idx[:4000]:
        assert oracle.bf16_value(int(i)) == float(ref[i])

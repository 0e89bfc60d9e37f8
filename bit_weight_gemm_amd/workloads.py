"""Seeded synthetic inputs for the fused NVFP4 + binary low-rank product.

This module only draws random operands and lays them out; it holds none of
the method's arithmetic (no quantiser, no packing of signs, no product).  The
rounding of drawn floats to bf16 and E4M3 uses torch's own casts (round to
nearest even), so neither the HIP path nor the oracle is involved in making
an input.  Both sides of every parity check start from these arrays.

Recipe (fixed draw order, so the r = 0 run shares x and R with the r > 0 run):
  1. rng = numpy.random.default_rng(seed)
  2. x = bf16(rng.standard_normal((M, K), float32))
  3. outliers only: idx = rng.choice(K, floor(0.01 K), replace=False);
     x[:, idx] = bf16(20 * rng.standard_normal((M, len(idx)), float32))
  4. R codes = rng.integers(0, 16, (N, K), dtype=uint8)   (uniform over 16 codes)
  5. R scales = max(E4M3(0.5 * |rng.standard_normal((N, K/16), float32)|), 2^-6)
     global scale g = float32(0.01)
  6. U = 1 - 2 * rng.integers(0, 2, (N, r), dtype=int8)
     V = 1 - 2 * rng.integers(0, 2, (K, r), dtype=int8)
  7. alpha_i = bf16(c * i^-0.5), i = 1..r

Start signs of the sign-peeling decomposition (make_start_signs): uint32
  words rng.integers(0, 2^32, (r, ceil(n/32))), bits >= n cleared; every
  bit is an independent fair coin (a set bit meaning -1).

Weights with planted sign structure (make_planted_weight): fp32
  W = sum_{l<L} decay^-l u_l v_l^T + noise * N(0,1), u_l, v_l i.i.d. fair
  +-1 (the case where peeling has clear sign decisions to make).

Residual matrices for the weight quantiser (make_residual): fp32
  w = sigma * rng.standard_normal((N, K), float32), and with outliers
  floor(0.01 K) columns (rng.choice) scaled by 20, the heavy-tailed input
  channels of a language-model layer.
"""
from __future__ import annotations

import numpy as np
import torch

# Decode shapes of the benchmark (M = decode batch, K = in-features,
# N = out-features, r = binary rank).
CONFIGS = {
    0: dict(name="tiny M1 K256 N256 r16", M=1, K=256, N=256, r=16, seed=0, c=0.05, outliers=False),
    1: dict(name="decode M1 K5120 N5120 r512", M=1, K=5120, N=5120, r=512, seed=1, c=0.05,
            outliers=False),
    2: dict(name="decode M8 K5120 N13824 r512 (1% outlier channels)", M=8, K=5120, N=13824,
            r=512, seed=2, c=0.05, outliers=True),
    3: dict(name="decode M32 K13824 N5120 r512", M=32, K=13824, N=5120, r=512, seed=3, c=0.05,
            outliers=False),
    4: dict(name="decode M32 K8192 N8192 r1024", M=32, K=8192, N=8192, r=1024, seed=4, c=0.03,
            outliers=False),
}

E4M3_MIN_SCALE_BYTE = 0x08  # 2^-6 as an E4M3 byte (exponent field 1, mantissa 0)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def to_e4m3_bytes(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[rows][K] codes 0..15 -> [rows][K/2] bytes, even k in the low nibble."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def make_inputs(M: int, K: int, N: int, r: int, seed: int, c: float = 0.05,
                outliers: bool = False, g: float = 0.01) -> dict:
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    if outliers:
        n_out = int(np.floor(0.01 * K))
        idx = rng.choice(K, n_out, replace=False)
        x[:, idx] = to_bf16_bits(20.0 * rng.standard_normal((M, n_out), dtype=np.float32))
    wcode = rng.integers(0, 16, (N, K), dtype=np.uint8)
    ws = to_e4m3_bytes(0.5 * np.abs(rng.standard_normal((N, K // 16), dtype=np.float32)))
    ws = np.maximum(ws, np.uint8(E4M3_MIN_SCALE_BYTE))
    if r > 0:
        U = (1 - 2 * rng.integers(0, 2, (N, r), dtype=np.int8)).astype(np.int8)
        V = (1 - 2 * rng.integers(0, 2, (K, r), dtype=np.int8)).astype(np.int8)
        i = np.arange(1, r + 1, dtype=np.float64)
        alpha = to_bf16_bits((c * i ** -0.5).astype(np.float32))
    else:
        U = np.zeros((N, 0), np.int8)
        V = np.zeros((K, 0), np.int8)
        alpha = np.zeros((0,), np.uint16)
    return dict(M=M, K=K, N=N, r=r, x=x, wcode=wcode, wcodes_packed=pack_nibbles(wcode),
                wscales=ws, g=np.float32(g), U=U, V=V, alpha=alpha)


def make_residual(N: int, K: int, seed: int, sigma: float = 0.02,
                  outliers: bool = False) -> np.ndarray:
    """Seeded fp32 residual R [N][K] for the NVFP4 weight quantiser."""
    rng = np.random.default_rng(seed)
    w = (sigma * rng.standard_normal((N, K), dtype=np.float32)).astype(np.float32)
    if outliers:
        idx = rng.choice(K, max(1, int(np.floor(0.01 * K))), replace=False)
        w[:, idx] *= np.float32(20.0)
    return w


def make_planted_weight(m: int, n: int, L: int, decay: float, seed: int,
                        noise: float = 1e-3) -> np.ndarray:
    rng = np.random.default_rng(seed)
    U = np.where(rng.random((m, L)) < 0.5, -1.0, 1.0)
    V = np.where(rng.random((n, L)) < 0.5, -1.0, 1.0)
    c = decay ** -np.arange(L, dtype=np.float64)
    W = (U * c) @ V.T + noise * rng.standard_normal((m, n))
    return W.astype(np.float32)


def make_start_signs(r: int, n: int, seed: int) -> np.ndarray:
    """uint32 [r][ceil(n/32)] random sign words for the peel's start vectors."""
    rng = np.random.default_rng(seed)
    nw = (n + 31) // 32
    w = rng.integers(0, 2 ** 32, (r, nw), dtype=np.uint64).astype(np.uint32)
    rem = n - 32 * (nw - 1)
    if rem < 32:
        w[:, -1] &= np.uint32((1 << rem) - 1)
    return w


def make_config(idx: int, r: int | None = None) -> dict:
    cfg = CONFIGS[idx]
    rr = cfg["r"] if r is None else r
    d = make_inputs(cfg["M"], cfg["K"], cfg["N"], rr, cfg["seed"], cfg["c"], cfg["outliers"])
    d["config"] = idx
    d["name"] = cfg["name"] if r is None else cfg["name"].replace(f"r{cfg['r']}", f"r{rr}")
    return d

"""Greedy sign peeling and the joint coefficient refit, in fp64 (numpy).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the HIP library
never imports or calls it.

Source: "BiLoCo: Binary Low-Rank Corrections for Post-Training Quantization"
(project README), intro (W ~ U diag(alpha) V^T + R, U in {+-1}^{m x r},
V in {+-1}^{n x r}) and section "Decomposition": every rank-one term starts
from random signs, alternates u = sign(R v) and v = sign(R^T u) for T steps,
takes the coefficient that minimises the Frobenius norm of the deflated
residual and deflates it; after all r terms the r coefficients are refit
together by least squares with the signs held fixed.

Readings where the pages leave a step open:
  * the random start is v (the first update is u = sign(R v)); its signs are
    an input (``v_init``), so both implementations start from the same draw;
  * one step is the pair of updates (u, then v); T steps per term;
  * sign(0) = +1;
  * the Frobenius-optimal coefficient for fixed u, v is u^T R v / (m n)
    (|u|^2 = m, |v|^2 = n);
  * the refit solves the normal equations G a = b with
    G_ij = (u_i . u_j)(v_i . v_j) and b_i = u_i^T W v_i, and the returned
    residual is W - U diag(a) V^T with the refit coefficients;
  * if the r sign outer products are linearly dependent (G singular, e.g. a
    term found twice), least squares has many minimisers; the oracle returns
    the one of minimum norm (the pseudo-inverse solution of G a = b, equal to
    the minimum-norm least-squares solution of the explicit design matrix,
    since b lies in the range of G).

Matrix products (numpy @) and the linear solves of the refit (numpy.linalg
solve, and lstsq for a singular G) are the only library primitives used.
"""
from __future__ import annotations

import numpy as np


def sign_pm1(x: np.ndarray) -> np.ndarray:
    """+1 where x >= 0 (zero included), -1 elsewhere."""
    return np.where(x >= 0, 1.0, -1.0)


def unpack_bits_pm1(words: np.ndarray, n: int) -> np.ndarray:
    """uint32 words [rows][ceil(n/32)] -> +-1 float64 [rows][n]; bit b of word w is
    coordinate 32w+b, a set bit meaning -1."""
    w = np.ascontiguousarray(words, dtype=np.uint32)
    bits = (w[:, :, None] >> np.arange(32, dtype=np.uint32)[None, None, :]) & 1
    bits = bits.reshape(w.shape[0], -1)[:, :n]
    return 1.0 - 2.0 * bits.astype(np.float64)


def peel(W: np.ndarray, r: int, T: int, v_init: np.ndarray, trace: bool = False) -> dict:
    """W: [m][n]; v_init: +-1 [r][n] (start signs of each term).

    Returns dict(U [m][r], V [n][r], alpha_greedy [r], alpha [r] (refit),
    R [m][n] (W - U diag(alpha) V^T), and with ``trace`` the per-term
    residual norms, the bilinear value u^T R v after every half step and the
    smallest |R v|, |R^T u| entry met by a sign decision relative to the row
    or column 1-norm of R (the decision margins)."""
    Wd = np.asarray(W, dtype=np.float64)
    m, n = Wd.shape
    R = Wd.copy()
    U = np.zeros((m, r))
    V = np.zeros((n, r))
    ag = np.zeros(r)
    norms = [float(np.sum(R * R))]
    bil = []
    margin = np.inf
    for i in range(r):
        v = np.asarray(v_init[i], dtype=np.float64)
        seq = []
        for _ in range(T):
            s = R @ v
            u = sign_pm1(s)
            if trace:
                margin = min(margin, float(np.min(np.abs(s) / np.abs(R).sum(axis=1).clip(1e-300))))
                seq.append(float(u @ s))
            t = R.T @ u
            v = sign_pm1(t)
            if trace:
                margin = min(margin, float(np.min(np.abs(t) / np.abs(R).sum(axis=0).clip(1e-300))))
                seq.append(float(v @ t))
        a = float(u @ R @ v) / (m * n)
        R -= a * np.outer(u, v)
        U[:, i], V[:, i], ag[i] = u, v, a
        if trace:
            norms.append(float(np.sum(R * R)))
            bil.append(seq)
    G = (U.T @ U) * (V.T @ V)
    b = np.einsum("ai,ai->i", U, Wd @ V)
    if np.linalg.matrix_rank(G) < r:
        # singular values below matrix_rank's own tolerance count as zero
        alpha = np.linalg.lstsq(G, b, rcond=r * np.finfo(np.float64).eps)[0]
    else:
        alpha = np.linalg.solve(G, b)
    out = {"U": U, "V": V, "alpha_greedy": ag, "alpha": alpha,
           "R": Wd - (U * alpha[None, :]) @ V.T}
    if trace:
        out.update(norms=np.array(norms), bilinear=bil, margin=margin)
    return out

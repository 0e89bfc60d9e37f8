"""GPU sign peeling (biloco_peel_decompose) against the fp64 oracle.

Where every sign decision of the oracle's run has a clear margin (planted
sign structure), the GPU must find the same signs bit for bit and the same
coefficients and residual to fp32 accuracy.  Where the terms come out
linearly dependent (a term found twice), least squares has many minimisers:
the GPU drops the repeated terms from the solve (coefficient 0), the oracle
returns the minimum-norm minimiser, so the refit is checked for what makes
it a minimiser (the normal equations and the residual norm).  On plain
random weights, up to the full decode weight shape, the decisions are not all
clear, so the GPU result is checked for what defines it, term by term from
its own earlier terms: each v is the sign of R^T u wherever that is clear of
rounding, each greedy coefficient is u^T R v / (m n), the refit solves the
normal equations of its signs, and the residual is W - U diag(alpha) V^T.
"""
import numpy as np
import pytest
import torch

from oracle import peel as P
from bit_weight_gemm_amd import binding as B
from bit_weight_gemm_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _unpack_cols(words: np.ndarray, r: int) -> np.ndarray:
    """[ceil(r/32)][len] words -> +-1 [len][r]."""
    w = np.ascontiguousarray(words).view(np.uint32)
    bits = (w[:, :, None] >> np.arange(32, dtype=np.uint32)[None, None, :]) & 1   # [RW][len][32]
    bits = bits.transpose(1, 0, 2).reshape(w.shape[1], -1)[:, :r]
    return 1.0 - 2.0 * bits.astype(np.float64)


def _gpu_peel(W: np.ndarray, r: int, T: int, vi: np.ndarray):
    Wt = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).cuda()
    vt = torch.from_numpy(np.ascontiguousarray(vi).view(np.int32)).cuda()
    o = B.biloco_peel_decompose(Wt, r, T, vt)
    torch.cuda.synchronize()
    m, n = W.shape
    return {"U": _unpack_cols(o["u_packed"].cpu().numpy(), r),
            "V": _unpack_cols(o["v_packed"].cpu().numpy(), r),
            "alpha": o["alpha"].cpu().numpy().astype(np.float64),
            "alpha_greedy": o["alpha_greedy"].cpu().numpy().astype(np.float64),
            "R": o["R"].cpu().numpy().astype(np.float64),
            "u_words": o["u_packed"].cpu().numpy().view(np.uint32),
            "v_words": o["v_packed"].cpu().numpy().view(np.uint32)}


# (m, n, r, T, planted terms, decay, seed): oracle margins >= 1e-3 of the row /
# column 1-norm at every decision; the second case's terms are dependent
PLANTED = [(96, 128, 6, 3, 8, 2.0, 5), (96, 128, 6, 3, 8, 4.0, 2), (100, 92, 5, 2, 8, 2.0, 1),
           (37, 260, 4, 4, 6, 3.0, 3)]


@pytest.mark.parametrize("case", PLANTED, ids=lambda c: "x".join(map(str, c[:4])) + f"-s{c[6]}")
def test_planted_exact(case):
    m, n, r, T, L, decay, seed = case
    W = wl.make_planted_weight(m, n, L, decay, seed)
    vi = wl.make_start_signs(r, n, 100 + seed)
    ref = P.peel(W.astype(np.float64), r, T, P.unpack_bits_pm1(vi, n), trace=True)
    assert ref["margin"] > 1e-3                   # every decision is clear of rounding
    g = _gpu_peel(W, r, T, vi)
    np.testing.assert_array_equal(g["U"], ref["U"])
    np.testing.assert_array_equal(g["V"], ref["V"])
    scale = np.abs(ref["alpha_greedy"]).max()
    np.testing.assert_allclose(g["alpha_greedy"], ref["alpha_greedy"], rtol=1e-5, atol=1e-6 * scale)
    U, V = ref["U"], ref["V"]
    G = (U.T @ U) * (V.T @ V)
    if np.linalg.matrix_rank(G) == r:
        np.testing.assert_allclose(g["alpha"], ref["alpha"], rtol=1e-5, atol=1e-6 * scale)
        tol = 1e-5 * (np.abs(W).max() + np.abs(ref["alpha"]).sum())
        assert np.abs(g["R"] - ref["R"]).max() <= tol
    else:
        _check_minimiser(W, g, ref)


def _check_minimiser(W, g, ref):
    """The GPU refit is a least-squares minimiser for the fixed signs: it
    solves the normal equations, its residual norm is the oracle's (the
    minimum), and the returned residual is W - U diag(alpha) V^T."""
    Wd = W.astype(np.float64)
    U, V = ref["U"], ref["V"]
    G = (U.T @ U) * (V.T @ V)
    b = np.einsum("ai,ai->i", U, Wd @ V)
    np.testing.assert_allclose(G @ g["alpha"], b, rtol=1e-5, atol=1e-5 * np.abs(b).max())
    res_gpu = np.sum((Wd - (U * g["alpha"]) @ V.T) ** 2)
    res_ref = np.sum(ref["R"] ** 2)
    assert res_gpu == pytest.approx(res_ref, rel=1e-5, abs=1e-6 * np.sum(Wd ** 2))
    Rref = Wd - (U * g["alpha"]) @ V.T
    assert np.abs(g["R"] - Rref).max() <= 1e-5 * (np.abs(W).max() + np.abs(g["alpha"]).sum())


def test_repeated_term_golden():
    """The hand-derived 4 x 4 case whose third term repeats the first: the
    signs and greedy coefficients are exact; the refit is a minimiser (the
    GPU drops the repeat: alpha = (33/32, 27/32, 0)); the greedy one is not."""
    import os
    vals = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "peel_repeated_term.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, rest = line.split(None, 1)
                vals[k] = np.array([float(t) for t in rest.split()])
    W = vals["W"].reshape(4, 4).astype(np.float32)
    signs = vals["v_init"].reshape(3, 4)
    vi = np.zeros((3, 1), np.uint32)
    for i in range(3):
        for k in range(4):
            if signs[i, k] < 0:
                vi[i, 0] |= np.uint32(1 << k)
    ref = P.peel(W.astype(np.float64), 3, 2, P.unpack_bits_pm1(vi, 4))
    g = _gpu_peel(W, 3, 2, vi)
    np.testing.assert_array_equal(g["U"].T.ravel(), vals["U"])
    np.testing.assert_array_equal(g["V"].T.ravel(), vals["V"])
    np.testing.assert_array_equal(g["alpha_greedy"], vals["alpha_greedy"])
    _check_minimiser(W, g, ref)
    np.testing.assert_allclose(g["alpha"], [33 / 32, 27 / 32, 0.0], rtol=0, atol=1e-6)


def _check_properties(W, r, T, g, terms):
    m, n = W.shape
    Wd = W.astype(np.float64)
    U, V, ag, al = g["U"], g["V"], g["alpha_greedy"], g["alpha"]
    # sign words beyond r are clear
    RW = (r + 31) // 32
    if r % 32:
        assert not np.any(g["u_words"][RW - 1] >> np.uint32(r % 32))
        assert not np.any(g["v_words"][RW - 1] >> np.uint32(r % 32))
    colw = np.abs(Wd).sum(axis=0)
    for i in terms:
        Ri = Wd - (U[:, :i] * ag[:i]) @ V[:, :i].T
        t = Ri.T @ U[:, i]
        tol = 1e-5 * (colw + m * np.abs(ag[:i]).sum())
        clear = np.abs(t) > tol
        np.testing.assert_array_equal(V[clear, i], np.where(t[clear] >= 0, 1.0, -1.0),
                                      err_msg=f"term {i}")
        a_ref = U[:, i] @ Ri @ V[:, i] / (m * n)
        assert ag[i] == pytest.approx(a_ref, rel=1e-4, abs=1e-6 * np.abs(ag).max()), i
    G = (U.T @ U) * (V.T @ V)
    b = np.einsum("ai,ai->i", U, Wd @ V)
    if np.linalg.matrix_rank(G) == r:
        a_ref = np.linalg.solve(G, b)
        np.testing.assert_allclose(al, a_ref, rtol=1e-4, atol=1e-5 * np.abs(a_ref).max())
    else:
        np.testing.assert_allclose(G @ al, b, rtol=1e-4, atol=1e-5 * np.abs(b).max())
    rows = np.unique(np.linspace(0, m - 1, min(m, 64)).astype(int))
    Rref = Wd[rows] - (U[rows] * al) @ V.T
    assert np.abs(g["R"][rows] - Rref).max() <= 1e-5 * (np.abs(W).max() + np.abs(al).sum())
    err_refit = np.sum((Wd - (U * al) @ V.T) ** 2)
    err_greedy = np.sum((Wd - (U * ag) @ V.T) ** 2)
    assert err_refit <= err_greedy * (1 + 1e-6)


@pytest.mark.parametrize("m,n,r,T", [(64, 96, 12, 2), (33, 44, 40, 3), (1, 4, 1, 1), (200, 36, 1, 5)])
def test_random_properties_small(m, n, r, T):
    W = wl.make_residual(m, n, seed=m * 7 + n, outliers=n >= 64)
    vi = wl.make_start_signs(r, n, seed=m + n)
    g = _gpu_peel(W, r, T, vi)
    _check_properties(W, r, T, g, range(r))


def test_full_weight_shape():
    m = n = 5120
    r, T = 512, 5
    W = wl.make_residual(m, n, seed=2024, outliers=True)
    vi = wl.make_start_signs(r, n, seed=77)
    print("peel 5120 x 5120, r 512, T 5", flush=True)
    g = _gpu_peel(W, r, T, vi)
    _check_properties(W, r, T, g, [0, 1, 17, 255, 511])

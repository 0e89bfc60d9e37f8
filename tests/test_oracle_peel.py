"""Pins of the sign-peeling oracle (greedy terms + joint refit).

* a hand-derived two-term decomposition (golden file);
* exact recovery of a planted rank-one sign matrix;
* each half step is the best sign vector for the other one fixed (brute
  force over every sign vector of a tiny matrix), so the bilinear value
  never decreases inside a term;
* every deflation lowers |R|^2 by exactly m n alpha^2 (the coefficient is the
  Frobenius optimum), so the residual never grows;
* the refit equals numpy's least-squares solve on the explicit design matrix
  of the r sign outer products, and is never worse than the greedy
  coefficients;
* with a term found twice (singular normal equations, golden file), the
  refit is the minimum-norm least-squares minimiser, derived by hand, where
  the greedy coefficients are not a minimiser at all.
"""
import itertools
import os

import numpy as np
import pytest

from oracle import peel as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name="peel_two_terms.txt"):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, rest = line.split(None, 1)
                d[k] = np.array([float(t) for t in rest.split()])
    return d


@pytest.mark.parametrize("T", [1, 3])
def test_golden_two_terms(T):
    g = _golden()
    W = g["W"].reshape(4, 4)
    o = P.peel(W, 2, T, g["v_init"].reshape(2, 4))
    np.testing.assert_array_equal(o["U"].T.ravel(), g["U"])
    np.testing.assert_array_equal(o["V"].T.ravel(), g["V"])
    np.testing.assert_allclose(o["alpha_greedy"], g["alpha"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["alpha"], g["alpha"], rtol=0, atol=1e-12)
    assert np.abs(o["R"]).max() < 1e-12


def _signs(rng, *shape):
    return np.where(rng.random(shape) < 0.5, -1.0, 1.0)


def test_planted_rank_one_is_recovered():
    rng = np.random.default_rng(1)
    m, n = 37, 52
    u, v = _signs(rng, m), _signs(rng, n)
    W = -0.8125 * np.outer(u, v)
    vi = _signs(rng, 1, n)
    assert vi[0] @ v != 0
    o = P.peel(W, 1, 1, vi)
    np.testing.assert_array_equal(np.outer(o["U"][:, 0], o["V"][:, 0]), np.outer(u, v) * np.sign(
        o["alpha_greedy"][0] / -0.8125))
    assert abs(abs(o["alpha_greedy"][0]) - 0.8125) < 1e-12
    assert np.abs(o["R"]).max() < 1e-12


def test_half_steps_are_brute_force_optima():
    rng = np.random.default_rng(2)
    m, n = 7, 5                         # not square: a transposed product would not even run
    W = rng.standard_normal((m, n))
    vi = _signs(rng, 1, n)
    o = P.peel(W, 1, 1, vi, trace=True)
    all_u = np.array(list(itertools.product([-1.0, 1.0], repeat=m)))
    all_v = np.array(list(itertools.product([-1.0, 1.0], repeat=n)))
    s = W @ vi[0]
    best_u = all_u[np.argmax(all_u @ s)]
    np.testing.assert_array_equal(o["U"][:, 0], best_u)
    assert o["bilinear"][0][0] == pytest.approx(np.max(all_u @ s), rel=1e-12)
    t = W.T @ best_u
    best_v = all_v[np.argmax(all_v @ t)]
    np.testing.assert_array_equal(o["V"][:, 0], best_v)
    # and the greedy coefficient is u^T W v / (m n)
    assert o["alpha_greedy"][0] == pytest.approx(best_u @ W @ best_v / (m * n), rel=1e-12)


def test_sign_of_zero_is_plus_one():
    W = np.zeros((3, 4))
    W[0, 0] = 1.0
    o = P.peel(W, 1, 1, np.array([[1.0, -1.0, 1.0, -1.0]]))
    # R v = (1, 0, 0): rows 1 and 2 are exact zeros -> +1
    np.testing.assert_array_equal(o["U"][:, 0], [1.0, 1.0, 1.0])


def test_monotone_steps_and_exact_deflation():
    rng = np.random.default_rng(3)
    m, n, r, T = 48, 40, 12, 4
    W = rng.standard_normal((m, n))
    o = P.peel(W, r, T, _signs(rng, r, n), trace=True)
    for seq in o["bilinear"]:
        assert all(b2 >= b1 - 1e-9 for b1, b2 in zip(seq, seq[1:]))
    norms = o["norms"]
    np.testing.assert_allclose(norms[:-1] - norms[1:], m * n * o["alpha_greedy"] ** 2,
                               rtol=1e-9, atol=1e-9)
    assert np.all(np.diff(norms) <= 1e-9)


def test_refit_is_least_squares():
    rng = np.random.default_rng(4)
    m, n, r = 30, 26, 6
    W = rng.standard_normal((m, n))
    o = P.peel(W, r, 3, _signs(rng, r, n))
    U, V = o["U"], o["V"]
    A = np.stack([np.outer(U[:, i], V[:, i]).ravel() for i in range(r)], axis=1)
    ref, *_ = np.linalg.lstsq(A, W.ravel(), rcond=None)
    np.testing.assert_allclose(o["alpha"], ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(o["R"], W - (U * o["alpha"]) @ V.T, atol=1e-12)
    greedy_err = np.sum((W - (U * o["alpha_greedy"]) @ V.T) ** 2)
    assert np.sum(o["R"] ** 2) <= greedy_err + 1e-12
    assert not np.allclose(o["alpha"], o["alpha_greedy"])      # the refit moved them


def test_unpack_bits():
    words = np.array([[0b1011, 0x80000000]], np.uint32)
    s = P.unpack_bits_pm1(words, 40)
    assert s.shape == (1, 40)
    np.testing.assert_array_equal(s[0, :4], [-1, -1, 1, -1])
    assert np.all(s[0, 4:32] == 1) and np.all(s[0, 32:] == 1)
    s2 = P.unpack_bits_pm1(words, 64)
    assert s2[0, 63] == -1


def test_repeated_term_refit_is_min_norm_least_squares():
    g = _golden("peel_repeated_term.txt")
    W = g["W"].reshape(4, 4)
    o = P.peel(W, 3, 2, g["v_init"].reshape(3, 4))
    np.testing.assert_array_equal(o["U"].T.ravel(), g["U"])
    np.testing.assert_array_equal(o["V"].T.ravel(), g["V"])
    np.testing.assert_array_equal(o["alpha_greedy"], g["alpha_greedy"])       # dyadic, exact
    # the design matrix has two equal columns
    U, V = o["U"], o["V"]
    A = np.stack([np.outer(U[:, i], V[:, i]).ravel() for i in range(3)], axis=1)
    assert np.linalg.matrix_rank(A) == 2
    np.testing.assert_allclose(o["alpha"], g["alpha"], rtol=0, atol=1e-12)
    # the same through another route: lstsq on the explicit design matrix
    ref, *_ = np.linalg.lstsq(A, W.ravel(), rcond=None)
    np.testing.assert_allclose(o["alpha"], ref, rtol=0, atol=1e-12)
    res_ls = float(np.sum(o["R"] ** 2))
    res_greedy = float(np.sum((W - (U * o["alpha_greedy"]) @ V.T) ** 2))
    assert res_ls == pytest.approx(g["resid_ls"][0], rel=0, abs=1e-12)
    assert res_greedy == pytest.approx(g["resid_greedy"][0], rel=0, abs=1e-12)
    assert res_ls < res_greedy - 0.5                 # greedy is not a minimiser here

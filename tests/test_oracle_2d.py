"""Pins of the oracle's two-sided rounding (GPTQ-2D) against the vectorized
one-sided definition (Theorem 2), a different topological order (Theorem 1),
the one-sided reductions (B = I, A = I), an independently written Babai
nearest-plane on the integer lattice, the identity metric and the
objective identity.  CPU only.
"""
import numpy as np
import pytest

from oracle import gptq_ref as o


def _spd(k, seed, lo=0.2, hi=3.0):
    r = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(r.standard_normal((k, k)))
    return (Q * r.uniform(lo, hi, k)) @ Q.T


def _problem(m, n, seed, scale=3.0):
    G, H = _spd(m, seed), _spd(n, seed + 100)
    X = np.random.default_rng(seed + 200).normal(0.0, scale, (m, n))
    return X, G, H, o.factor_u(G), o.factor_u(H)


@pytest.mark.parametrize("m,n,qmin,qmax", [(5, 7, -8, 7), (9, 4, -8, 7), (13, 13, -8, 7), (6, 10, 0, 3),
                                           (1, 9, -8, 7), (8, 1, -2, 2)])
def test_anti_diagonal_equals_vectorized_sweep(m, n, qmin, qmax):
    # [2D] Theorem 2: the cubic anti-diagonal algorithm reproduces the 1D
    # sweep over vec(X) with the Kronecker Gram exactly
    X, G, H, UG, UH = _problem(m, n, m * 31 + n)
    a = o.round_2d(X, UG, UH, qmin, qmax)
    b = o.round_2d_vectorized(X, UG, UH, qmin, qmax)
    assert np.array_equal(a["Z"], b["Z"])
    assert np.abs(a["E"] - b["E"]).max() <= 1e-9 * max(1.0, np.abs(b["E"]).max())
    assert a["Z"].min() >= qmin and a["Z"].max() <= qmax


def test_row_major_order_gives_the_same_rounding():
    # [2D] Theorem 1: any order respecting the dependencies gives the same
    # result; the row-major order is the 1D sweep over vec(X^T) with
    # UG kron UH
    X, G, H, UG, UH = _problem(7, 6, 5)
    r = o.round_1d(X.ravel(), np.kron(UG, UH), -8, 7)
    a = o.round_2d(X, UG, UH, -8, 7)
    assert np.array_equal(r["z"].reshape(7, 6), a["Z"])


def test_one_sided_reductions():
    # B = I: every column is rounded on its own against G; A = I: every row
    # against H ([2D] section 5: one-sided rounding is the case B = I)
    X, G, H, UG, UH = _problem(6, 8, 11)
    a = o.round_2d(X, UG, np.eye(8), -8, 7)
    for j in range(8):
        assert np.array_equal(a["Z"][:, j], o.round_1d(X[:, j], UG, -8, 7)["z"])
    b = o.round_2d(X, np.eye(6), UH, -8, 7)
    for i in range(6):
        assert np.array_equal(b["Z"][i], o.round_1d(X[i], UH, -8, 7)["z"])


def test_one_sided_rounding_is_babai_nearest_plane():
    # round_1d against an independently written nearest-plane solver on the
    # lattice with Gram K = L^T L (L lower, the QL factor): coordinate p is
    # rounded at c_p = x_p + L[p, :p] (x - z)[:p] / L[p, p]
    rng = np.random.default_rng(12)
    for N in (5, 11, 17):
        K = _spd(N, N)
        x = rng.normal(0, 4, N)
        L = o.ql_lower_from_gram(K)
        assert np.allclose(L.T @ L, K)
        z = np.zeros(N)
        for p in range(N):
            c = x[p] + L[p, :p] @ (x - z)[:p] / L[p, p]
            z[p] = np.clip(np.rint(np.float32(c)), -8, 7)
        r = o.round_1d(x, o.factor_u(K), -8, 7)
        assert np.array_equal(r["z"], z)


def test_identity_metric_is_round_to_nearest():
    X, _, _, _, _ = _problem(5, 6, 13)
    a = o.round_2d(X, np.eye(5), np.eye(6), -8, 7)
    assert np.array_equal(a["Z"], np.clip(np.rint(X.astype(np.float32)), -8, 7))


def test_objective_identity():
    # sum of squared scaled errors = ||A (Z - X) B||_F^2 with the Grams
    # formed directly (no factor involved)
    rng = np.random.default_rng(14)
    m, n = 7, 9
    A = rng.normal(size=(m, m)) + 3 * np.eye(m)
    B = rng.normal(size=(n, n)) + 3 * np.eye(n)
    G, H = A.T @ A, B @ B.T
    X = rng.normal(0, 3, (m, n))
    a = o.round_2d(X, o.factor_u(G), o.factor_u(H), -8, 7)
    direct = float(np.sum((A @ (a["Z"] - X) @ B) ** 2))
    assert a["J"] == pytest.approx(direct, rel=1e-10)
    assert o.objective_2d(X, a["Z"], G, H) == pytest.approx(direct, rel=1e-10)

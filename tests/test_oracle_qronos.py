"""Pins of the oracle's quantised-input target: the X_q = X reduction, the
completed-square identity with random codes, an independent least-squares
route to the target, the Babai nearest-plane solver on the target, and the
cross Gram against a direct product.  CPU only.
"""
import numpy as np
import pytest

from oracle import gptq_ref as o
from test_oracle_pins import _spd_problem, _to_bf16_bits


def _perturbed(X_bits, seed, scale=0.05):
    """A seeded stand-in for the inputs of an already-quantised network."""
    X = o.bf16_bits_to_f64(X_bits)
    r = np.random.default_rng(seed)
    return _to_bf16_bits((X + scale * X.std() * r.standard_normal(X.shape)).astype(np.float32))


def test_cross_gram_is_the_product():
    X, _ = _spd_problem(51, 24)
    Xq = _perturbed(X, 1)
    A, B = o.bf16_bits_to_f64(Xq), o.bf16_bits_to_f64(X)
    G = o.cross_gram(Xq, X, chunk=7)
    assert np.abs(G - A.T @ B).max() <= 1e-12 * np.abs(A.T @ B).max()
    assert np.allclose(o.cross_gram(X, X), o.hessian(X), rtol=1e-14, atol=0)


def test_same_inputs_reduce_to_gptq():
    X, W = _spd_problem(52, 32, out=8)
    a = o.gptq_qronos(W, X, X, 3, 8, 16, lam_rel=0.01)
    b = o.gptq_layer(W, X, 3, 8, 16, lam_rel=0.01)
    assert np.abs(a["W_target"] - W).max() <= 1e-12 * np.abs(W).max()
    assert np.array_equal(a["codes"], b["codes"])


def test_completed_square_identity():
    # ||Xq q - X w||^2 + lam ||q - w||^2 - (q - w*)^T Hq_lam (q - w*) is the
    # same for every q (it depends on w alone)
    X, W = _spd_problem(53, 20, out=1)
    Xq = _perturbed(X, 2)
    A, B = o.bf16_bits_to_f64(Xq), o.bf16_bits_to_f64(X)
    Hq, G = A.T @ A, A.T @ B
    lam = 0.3
    w = W[0]
    ws = o.qronos_target(W, Hq, G, lam)[0]
    Hl = Hq + lam * np.eye(20)
    r = np.random.default_rng(3)
    consts = []
    for _ in range(6):
        q = r.normal(0, 0.05, 20)
        direct = np.sum((A @ q - B @ w) ** 2) + lam * np.sum((q - w) ** 2)
        consts.append(direct - (q - ws) @ Hl @ (q - ws))
    assert np.ptp(consts) <= 1e-9 * max(abs(c) for c in consts)


def test_target_is_the_ridge_least_squares_solution():
    X, W = _spd_problem(54, 16, out=3)
    Xq = _perturbed(X, 4)
    A, B = o.bf16_bits_to_f64(Xq), o.bf16_bits_to_f64(X)
    lam = 0.2
    ws = o.qronos_target(W, A.T @ A, A.T @ B, lam)
    for i in range(3):
        Ms = np.vstack([A, np.sqrt(lam) * np.eye(16)])
        rhs = np.concatenate([B @ W[i], np.sqrt(lam) * W[i]])
        sol = np.linalg.lstsq(Ms, rhs, rcond=None)[0]
        assert np.abs(sol - ws[i]).max() <= 1e-9 * np.abs(ws[i]).max()


def test_codes_are_babai_on_the_target():
    X, W = _spd_problem(55, 24, out=5)
    Xq = _perturbed(X, 5)
    res = o.gptq_qronos(W, X, Xq, 3, 0, None, lam_rel=0.01)
    L = o.ql_lower_from_gram(res["Hq"] + res["lam"] * np.eye(24))
    bb = o.babai(res["W_target"], L, 3, 0)
    assert np.array_equal(bb["codes"], res["codes"])


def test_objective_decomposition():
    # J_q from the Grams equals ||Xq What^T - X W^T||^2 formed from the data
    X, W = _spd_problem(56, 16, out=4)
    Xq = _perturbed(X, 6)
    res = o.gptq_qronos(W, X, Xq, 4, 0, 8, lam_rel=0.01)
    A, B = o.bf16_bits_to_f64(Xq), o.bf16_bits_to_f64(X)
    direct = float(np.sum((A @ res["What"].T - B @ W.T) ** 2))
    assert res["J_q"] == pytest.approx(direct, rel=1e-9)

"""Pins of the oracle's refinement loop after the intrinsic LoRA (OLrC and
Bid-Up), against closed forms, an independent matrix-square-root route,
brute force over the grid, and decoupled special cases.  CPU only.
"""
import numpy as np
import pytest

from oracle import gptq_ref as o
from test_oracle_pins import _lowrank_problem, _rng, _spd_problem


def _quantized(seed, bits=3, group=0, n=48, out=10, lowrank=True):
    """A layer, its Hessian and a GPTQ result on it (the start of a refinement)."""
    if lowrank:
        X, W = _lowrank_problem(seed, n=n, out=out)
    else:
        X, W = _spd_problem(seed, n, out=out)
    H = o.hessian(X)
    Hl, _ = o.damp(H, lam_rel=1e-2)
    g = o.gptq_sweep(W, o.factor_u(Hl), bits, group, block=16)
    return W, H, g


def _J(W, What, C, H):
    D = W - What - C
    return float(np.sum((D @ H) * D))


# ------------------------------------------------------------------- OLrC ---
def test_olrc_identity_hessian_is_truncated_svd():
    # H = I: J(C) = ||E - C||_F^2, minimised by the rank-r truncated SVD of E
    rng = _rng(31)
    W = rng.standard_normal((9, 14))
    What = np.round(W * 2) / 2
    E = W - What
    U, s, Vt = np.linalg.svd(E, full_matrices=False)
    for r in (1, 3, 5):
        C_svd = (U[:, :r] * s[:r]) @ Vt[:r]
        res = o.olrc(W, What, np.eye(14), r)
        assert np.abs(res["C"] - C_svd).max() <= 1e-12 * np.abs(E).max()
        assert res["J"] == pytest.approx(float(np.sum(s[r:] ** 2)), rel=1e-10)


def test_olrc_equals_square_root_route():
    # C = [E S]_r S^{-1} with S = H^{1/2} (symmetric square root by eigh, the
    # truncation by SVD, then a solve): a different route to the same optimum
    W, H, g = _quantized(32)
    E = W - g["What"]
    lam, V = np.linalg.eigh(H)
    S = (V * np.sqrt(lam)) @ V.T
    U, s, Vt = np.linalg.svd(E @ S, full_matrices=False)
    for r in (2, 4, 6):
        ES_r = (U[:, :r] * s[:r]) @ Vt[:r]
        C_ref = np.linalg.solve(S.T, ES_r.T).T
        res = o.olrc(W, g["What"], H, r)
        assert np.abs(res["C"] - C_ref).max() <= 1e-7 * np.abs(C_ref).max()
        assert res["J"] == pytest.approx(float(np.sum(s[r:] ** 2)), rel=1e-8)
        # the factors: R_out orthonormal, C = R_out L^T
        assert np.abs(res["R_out"].T @ res["R_out"] - np.eye(r)).max() < 1e-12
        assert np.abs(res["R_out"] @ res["L"].T - res["C"]).max() <= 1e-12 * np.abs(E).max()


def test_olrc_beats_other_rank_r_corrections():
    W, H, g = _quantized(33)
    r = 4
    res = o.olrc(W, g["What"], H, r)
    rng = _rng(34)
    for _ in range(20):
        C = rng.standard_normal((W.shape[0], r)) @ rng.standard_normal((r, W.shape[1])) * 1e-3
        assert res["J"] <= _J(W, g["What"], res["C"] + C, H) + 1e-18
    # the ridge-optimal R for the fixed basis L = V_r (the LoRA's own
    # compensation for a fixed Q, lam -> 0) is one candidate among all rank r
    V = o.top_eigvecs(H, r)
    E = W - g["What"]
    K = V.T @ H @ V
    Rt = np.linalg.solve(K, V.T @ H @ E.T)
    assert res["J"] <= _J(W, g["What"], Rt.T @ V.T, H) * (1 + 1e-12)


# ----------------------------------------------------------------- Bid-Up ---
def _row_objective(w, c, what, H):
    d = w - c - what
    return float(d @ H @ d)


@pytest.mark.parametrize("bits,group,lowrank", [(3, 0, True), (2, 8, False), (4, 16, True)])
def test_bid_up_moves_are_coordinate_optimal_by_brute_force(bits, group, lowrank):
    # replay the pass one coordinate at a time, evaluating J_i for every grid
    # value directly (no vertex formula): the pass's choice must be a minimiser,
    # and it must stay put unless it strictly improves
    W, H, g = _quantized(35 + bits, bits, group, lowrank=lowrank)
    out, n = W.shape
    C = 1e-3 * _rng(36).standard_normal((out, 2)) @ _rng(37).standard_normal((2, n))
    bu = o.bid_up(W, C, g["codes"], g["scales"], g["zeros"], H, bits, group)
    maxq = (1 << bits) - 1
    gs = group if group else n
    codes = g["codes"].astype(np.int64).copy()
    S = np.repeat(g["scales"], gs, axis=1).astype(np.float32)
    Z = np.repeat(g["zeros"], gs, axis=1).astype(np.float32)
    moves = 0
    for i in range(out):
        for j in range(n):
            def what_of(q):
                row = codes[i].astype(np.float32).copy()
                row[j] = q
                return (S[i] * (row - Z[i])).astype(np.float32).astype(np.float64)
            vals = np.array([_row_objective(W[i], C[i], what_of(q), H) for q in range(maxq + 1)])
            cur = vals[codes[i, j]]
            chosen = int(bu["codes"][i, j])
            best = vals.min()
            assert vals[chosen] <= best + 1e-9 * max(1.0, abs(best)), (i, j)
            if chosen != codes[i, j]:
                assert vals[chosen] < cur
                moves += 1
            else:
                assert cur <= best + 1e-9 * max(1.0, abs(best))
            codes[i, j] = chosen
    assert moves == bu["moves"] and moves > 0
    assert np.array_equal(codes, bu["codes"])


def test_bid_up_decoupled_hessian_is_round_to_nearest():
    # diagonal H and C = 0: the coordinates decouple, so one pass from any
    # start lands every code on the grid point nearest w (what the sweep's
    # rounding gives on the fixed grid)
    rng = _rng(38)
    out, n, bits = 5, 24, 3
    W = rng.standard_normal((out, n))
    H = np.diag(rng.uniform(0.5, 2.0, n))
    maxq = (1 << bits) - 1
    s, r, z, _ = o.grid_fit(W, maxq)
    start = rng.integers(0, maxq + 1, (out, n)).astype(np.uint8)
    bu = o.bid_up(W, np.zeros_like(W), start, s[:, None], z[:, None], H, bits, 0)
    q, _, _ = o.quantize_values(W, s[:, None], r[:, None], z[:, None], maxq)
    assert np.array_equal(bu["codes"], q.astype(np.uint8))


def test_bid_up_objective_accounting_and_fixed_point():
    W, H, g = _quantized(39, 3, 8, lowrank=False)
    C = np.zeros_like(W)
    codes = g["codes"]
    J = o.objective(W, g["What"], H)
    for it in range(50):
        bu = o.bid_up(W, C, codes, g["scales"], g["zeros"], H, 3, 8)
        assert bu["J0"] == pytest.approx(J, rel=1e-10)
        assert bu["J"] == pytest.approx(bu["J0"] + bu["dJ"].sum(), rel=1e-9)
        assert bu["J"] <= bu["J0"]
        J = bu["J"]
        codes = bu["codes"]
        if bu["moves"] == 0:
            break
    assert bu["moves"] == 0 and it > 0
    # at the fixed point no single code change lowers any row's objective
    What = o.dequantize(codes, g["scales"], g["zeros"], 8)
    for i in range(W.shape[0]):
        base = _row_objective(W[i], 0.0, What[i], H)
        for j in range(W.shape[1]):
            for q in range(8):
                row = codes[i].astype(np.float32).copy()
                row[j] = q
                s = np.repeat(g["scales"][i], 8).astype(np.float32)
                z = np.repeat(g["zeros"][i], 8).astype(np.float32)
                wh = (s * (row - z)).astype(np.float32).astype(np.float64)
                assert _row_objective(W[i], 0.0, wh, H) >= base * (1 - 1e-12)


# ------------------------------------------------------------------- loop ---
def test_refine_trace_is_non_increasing_and_rank_zero_rounds_zero_is_lora():
    X, W = _lowrank_problem(40)
    H = o.hessian(X)
    res = o.lora_refine(W, H, 4, 3, 0, block=16, lam_rel=1e-4, rounds=3)
    tr = res["trace"]
    assert len(tr) == 2 * 3 + 2
    assert all(b <= a * (1 + 1e-12) for a, b in zip(tr, tr[1:]))
    assert res["trace"][-1] == pytest.approx(_J(W, res["What"], res["R_out"] @ res["L"].T, H), rel=1e-10)
    base = o.lora(W, H, 4, 3, 0, block=16, lam_rel=1e-4)
    zero = o.lora_refine(W, H, 4, 3, 0, block=16, lam_rel=1e-4, rounds=0)
    assert np.array_equal(zero["codes"], base["codes"]) and zero["trace"] == [base["J"]]


def test_refine_from_round_to_nearest_start_improves():
    # OLrC then Bid-Up from round-to-nearest codes on the same grid (not
    # coordinate-optimal under a correlated H): codes move, J drops each step
    W, H, g = _quantized(41, 3, 0, lowrank=False)
    s, r, z, _ = o.grid_fit(W, 7)
    q, What, _ = o.quantize_values(W, s[:, None], r[:, None], z[:, None], 7)
    oc = o.olrc(W, What, H, 4)
    bu = o.bid_up(W, oc["C"], q.astype(np.uint8), s[:, None], z[:, None], H, 3, 0)
    assert bu["moves"] > 0 and bu["J"] < oc["J"] <= o.objective(W, What, H)

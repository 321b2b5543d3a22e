"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: exact
rational arithmetic, closed forms, an independently written solver, brute
force, or a hand-worked fixture under tests/golden/.  None needs a GPU.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import gptq_ref as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest-even) and return the bit patterns."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _spd_problem(seed, n, tokens=None, decay=1.0, out=6):
    rng = _rng(seed)
    tokens = tokens or 4 * n
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    z = rng.standard_normal((tokens, n)) * (np.arange(1, n + 1) ** (-decay / 2))
    X = _to_bf16_bits((z @ Q.T).astype(np.float32))
    W = (0.02 * rng.standard_normal((out, n))).astype(np.float32).astype(np.float64)
    return X, W


# ---------------------------------------------------------------- inputs ---
def test_bf16_decode_known_patterns():
    bits = np.array([0x0000, 0x3F80, 0xC000, 0x3E80, 0x7F7F, 0x0001], dtype=np.uint16)
    v = o.bf16_bits_to_f64(bits)
    assert v[0] == 0.0 and v[1] == 1.0 and v[2] == -2.0 and v[3] == 0.25
    assert v[4] == (2 - 2 ** -7) * 2.0 ** 127
    assert v[5] == 2.0 ** -133  # smallest bf16 subnormal


# ---------------------------------------------------------------- a1 -------
def test_hessian_equals_exact_rational_sum():
    rng = _rng(1)
    tokens, n = 37, 5
    vals = rng.integers(-40, 41, size=(tokens, n)) / 8.0  # exact in bf16
    X = _to_bf16_bits(vals.astype(np.float32))
    H = o.hessian(X, chunk=7)
    for i in range(n):
        for j in range(n):
            exact = sum(Fraction(vals[t, i]) * Fraction(vals[t, j]) for t in range(tokens))
            assert H[i, j] == float(exact)


def test_hessian_order_and_accumulate():
    X, _ = _spd_problem(2, 24, tokens=300)
    H1 = o.hessian(X, chunk=2048)
    H2 = o.hessian(X[150:], chunk=13, H0=o.hessian(X[:150], chunk=64))
    Xf = o.bf16_bits_to_f64(X)
    Hs = np.array([[math.fsum(Xf[:, i] * Xf[:, j]) for j in range(24)] for i in range(24)])
    scale = np.abs(Hs).max()
    assert np.abs(H1 - Hs).max() <= 1e-13 * scale
    assert np.abs(H2 - Hs).max() <= 1e-13 * scale
    assert np.array_equal(H1, H1.T)


# ---------------------------------------------------------------- a2 -------
def test_damping_closed_form():
    H = np.diag([1.0, 2.0, 3.0, 6.0]) + 0.5  # mean diag = 3.5
    Hl, lam = o.damp(H, lam_abs=0.25, lam_rel=0.01)
    assert lam == pytest.approx(0.285, rel=1e-15)
    off = ~np.eye(4, dtype=bool)
    assert np.array_equal(Hl[off], H[off])
    assert np.allclose(np.diag(Hl) - np.diag(H), 0.285, rtol=1e-14)


# ---------------------------------------------------------------- a3 -------
@pytest.mark.parametrize("n,decay", [(8, 1.0), (40, 0.8), (96, 1.0)])
def test_factor_three_routes_agree(n, decay):
    X, _ = _spd_problem(3 + n, n, decay=decay)
    H = o.hessian(X)
    Hl, lam = o.damp(H, lam_rel=0.01)
    U1 = o.factor_u(Hl)
    U2 = o.factor_u_reversal(Hl)
    L = o.ql_lower_from_data(X, math.sqrt(lam))  # [X; mu I], data space
    U3 = np.linalg.inv(L).T
    L4 = o.ql_lower_from_gram(Hl)
    U4 = np.linalg.inv(L4).T
    sc = np.abs(U1).max()
    for U in (U2, U3, U4):
        assert np.abs(U - U1).max() <= 1e-9 * sc
    assert np.allclose(np.tril(U1, -1), 0) and (np.diag(U1) > 0).all()
    assert np.abs(U1 @ Hl @ U1.T - np.eye(n)).max() < 1e-9


def test_not_pd_raises_with_reversed_pivot_index():
    H = np.diag([1.0, 1.0, -1.0, 1.0])
    with pytest.raises(o.NotPositiveDefinite) as e:
        o.factor_u(H)
    assert e.value.info == 3  # eliminating from column 3 down, column 2 fails
    H = np.eye(5)
    H[1, 1] = 0.0
    with pytest.raises(o.NotPositiveDefinite) as e:
        o.factor_u_reversal(H)
    assert e.value.info == 2


# ---------------------------------------------------------------- grid -----
def test_grid_fit_properties():
    rng = _rng(5)
    for bits in (2, 3, 4, 8):
        maxq = 2 ** bits - 1
        v = rng.standard_normal((200, 16)) * rng.uniform(0.01, 3, size=(200, 1)) + rng.uniform(-1, 1, (200, 1))
        s, r, z, _ = o.grid_fit(v, maxq)
        lo = np.minimum(v.min(1), 0)
        hi = np.maximum(v.max(1), 0)
        assert np.allclose(s * maxq, hi - lo, rtol=1e-6)
        assert ((z >= 0) & (z <= maxq) & (z == np.round(z))).all()
        # 0 lies on the grid, and the grid ends lie within half a step of lo and hi
        assert np.allclose(-z * s, lo, atol=0.5 * s.max() * 1.0001 + 0)
        assert (np.abs(-z.astype(np.float64) * s - lo) <= 0.5001 * s).all()
        assert (np.abs((maxq - z.astype(np.float64)) * s - hi) <= 0.5001 * s).all()
    s, r, z, _ = o.grid_fit(np.zeros((1, 4)), 15)
    assert s[0] == 1 and z[0] == 0


def test_rounding_is_nearest_grid_point_by_brute_force():
    rng = _rng(6)
    for bits in (2, 3, 4):
        maxq = 2 ** bits - 1
        v = rng.standard_normal((64, 32))
        s, r, z, _ = o.grid_fit(v, maxq)
        w = v * 1.3  # some values fall outside the grid: clamping
        q, what, x = o.quantize_values(w, s[:, None], r[:, None], z[:, None], maxq)
        grid = s[:, None, None].astype(np.float64) * (np.arange(maxq + 1)[None, None, :] - z[:, None, None])
        dist = np.abs(w[:, :, None] - grid)
        best = dist.argmin(-1)
        srt = np.sort(dist, -1)
        clear = (srt[..., 1] - srt[..., 0]) > 1e-5 * s[:, None]
        assert np.array_equal(q[clear].astype(int), best[clear])


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_fp32_decisions_equal_plain_fp64_division_away_from_ties(bits):
    """The grid and code decisions, taken in float32 with a reciprocal
    multiply, equal the plain float64 definitions s = (hi - lo)/maxq,
    z = rne(-lo/s), q = clamp(rne(w/s + z)) everywhere except within the
    float32 rounding bound of a tie (|frac - 1/2| below a few ulps of the
    operands: under 8e-6 at 4 bits and 1.3e-4 at 8 bits for values inside
    the grid)."""
    rng = _rng(40 + bits)
    maxq = 2 ** bits - 1
    rows, g = 4000, 64
    V = rng.standard_normal((rows, g)) * 10.0 ** rng.uniform(-3, 1, (rows, 1))
    V[:100] = np.abs(V[:100])       # all-positive groups: lo = 0, z = 0
    V[100:200] = -np.abs(V[100:200])  # all-negative groups: hi = 0, z = maxq
    s, r, z, zraw = o.grid_fit(V, maxq)
    v32 = V.astype(np.float32).astype(np.float64)
    lo = np.minimum(v32.min(1), 0.0)
    hi = np.maximum(v32.max(1), 0.0)
    s64 = (hi - lo) / maxq
    u = 2.0 ** -24
    # the stored scale is the float64 scale to within two float32 roundings
    assert (np.abs(s.astype(np.float64) - s64) <= 2.001 * u * s64).all()
    # zero points: equal to rne(-lo/s) away from a tie
    x64 = -lo / s64
    z64 = np.clip(np.rint(x64), 0, maxq)
    bound = (x64 + 1.0) * 8 * u
    tie = np.abs(x64 - np.floor(x64) - 0.5) <= bound
    assert np.array_equal(z.astype(np.float64)[~tie], z64[~tie])
    # codes of the group's own values and of values past the grid's ends
    for w in (v32, 1.5 * v32 - 0.3 * s64[:, None]):
        q, what, x = o.quantize_values(w, s[:, None], r[:, None], z[:, None], maxq)
        xd = w / s64[:, None] + z[:, None].astype(np.float64)
        qd = np.clip(np.rint(xd), 0, maxq)
        bound = (3.0 * np.abs(w / s64[:, None]) + np.abs(xd) + 1.0) * 2 * u
        tie = np.abs(xd - np.floor(xd) - 0.5) <= bound
        assert np.array_equal(q.astype(np.float64)[~tie], qd[~tie])
        assert tie.mean() < 1e-3
        if w is v32:  # inside the grid: |w/s| and |x| at most maxq
            assert bound.max() <= (4 * maxq + 1) * 2 * u * 1.001
    # the decision's window is far inside the 1e-3 near-tie replay window of the parity tests
    assert bound.max() < 1e-3


# ---------------------------------------------------------------- sweep ----
@pytest.mark.parametrize("group", [0, 8])
def test_identity_hessian_reduces_to_round_to_nearest(group):
    rng = _rng(7)
    n, out, maxq = 32, 10, 15
    W = 0.02 * rng.standard_normal((out, n))
    Hl, _ = o.damp(3.7 * np.eye(n), lam_rel=0.01)
    res = o.gptq_sweep(W, o.factor_u(Hl), 4, group, block=8)
    g = group or n
    for k in range(n // g):
        blk = W[:, k * g:(k + 1) * g]
        s = res["scales"][:, k].astype(np.float64)
        z = res["zeros"][:, k].astype(np.float64)
        grid = s[:, None, None] * (np.arange(maxq + 1)[None, None, :] - z[:, None, None])
        best = np.abs(blk[:, :, None] - grid).argmin(-1)
        assert np.array_equal(res["codes"][:, k * g:(k + 1) * g], best)
    assert np.abs(res["W_final"] - W).max() == 0.0  # no compensation reaches anything


@pytest.mark.parametrize("group,bits", [(0, 4), (16, 3), (8, 2)])
def test_closed_form_identities(group, bits):
    X, W = _spd_problem(8, 48, out=12)
    H = o.hessian(X)
    Hl, lam = o.damp(H, lam_rel=0.01)
    U = o.factor_u(Hl)
    res = o.gptq_sweep(W, U, bits, group)
    D = W - res["What"]
    assert np.abs(D - res["E"] @ U).max() <= 1e-12 * max(1.0, np.abs(D).max())
    J_lam = np.sum((D @ Hl) * D)
    assert np.sum(res["E"] ** 2) == pytest.approx(J_lam, rel=1e-10)
    # the objective of the pages is the undamped one; J_lam - lam ||D||^2 = J
    J = o.objective(W, res["What"], H)
    assert J == pytest.approx(J_lam - lam * np.sum(D * D), rel=1e-9)


@pytest.mark.parametrize("group", [0, 8, 32])
def test_blocked_equals_unblocked(group):
    X, W = _spd_problem(9, 64, out=16)
    Hl, _ = o.damp(o.hessian(X), lam_rel=0.01)
    U = o.factor_u(Hl)
    ref = o.gptq_sweep(W, U, 3, group)
    for B in (1, 8, 32, 64, 128):
        if group and not (group % B == 0 or B % group == 0):
            continue
        res = o.gptq_sweep(W, U, 3, group, block=B)
        assert np.array_equal(res["codes"], ref["codes"]), B
        assert np.array_equal(res["zeros"], ref["zeros"]), B
        assert np.allclose(res["E"], ref["E"], rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("group,bits", [(0, 4), (8, 2), (16, 3)])
def test_gptq_equals_babai_nearest_plane(group, bits):
    X, W = _spd_problem(10, 48, out=20)
    H = o.hessian(X)
    Hl, lam = o.damp(H, lam_rel=0.01)
    g = o.gptq_sweep(W, o.factor_u(Hl), bits, group, block=16)
    L = o.ql_lower_from_data(X, math.sqrt(lam))  # data-space basis [X; mu I]
    b = o.babai(W, L, bits, group)
    assert np.array_equal(g["codes"], b["codes"])
    assert np.array_equal(g["zeros"], b["zeros"])
    assert np.allclose(g["scales"], b["scales"], rtol=1e-6)


@pytest.mark.parametrize("n", [3, 5, 8])
def test_brute_force_lower_bounds_gptq(n):
    rng = _rng(11 + n)
    maxq = 3
    for trial in range(6):
        A = rng.standard_normal((3 * n, n))
        H = A.T @ A
        Hl, _ = o.damp(H, lam_rel=0.05)
        w = 0.02 * rng.standard_normal((1, n))
        res = o.gptq_sweep(w, o.factor_u(Hl), 2, 0)
        s, z = float(res["scales"][0, 0]), float(res["zeros"][0, 0])
        best, _ = o.brute_force_row(w[0], Hl, s, z, maxq)
        D = w[0] - res["What"][0]
        J = D @ Hl @ D
        assert best <= J + 1e-15
    # diagonal H: the greedy sweep is optimal
    Hd = np.diag(rng.uniform(0.5, 2.0, n))
    w = 0.02 * rng.standard_normal((1, n))
    res = o.gptq_sweep(w, o.factor_u(Hd), 2, 0)
    s, z = float(res["scales"][0, 0]), float(res["zeros"][0, 0])
    best, _ = o.brute_force_row(w[0], Hd, s, z, maxq)
    D = w[0] - res["What"][0]
    assert D @ Hd @ D == pytest.approx(best, rel=1e-12, abs=1e-18)


def test_nearest_plane_error_bound():
    X, W = _spd_problem(12, 32, out=64)
    Hl, _ = o.damp(o.hessian(X), lam_rel=0.01)
    U = o.factor_u(Hl)
    res = o.gptq_sweep(0.3 * W, U, 4, 0)
    s = res["scales"][:, 0].astype(np.float64)
    D = 0.3 * W - res["What"]
    err = res["E"] * np.diag(U)[None, :]  # rounding error of each step
    ok = (np.abs(err) <= 0.5 * s[:, None] * (1 + 1e-5)).all(1)  # rows with no clamping
    assert ok.sum() > 10
    J = np.sum((D @ Hl) * D, axis=1)
    bound = 0.25 * s ** 2 * np.sum(1.0 / np.diag(U) ** 2)
    assert (J[ok] <= bound[ok] * (1 + 1e-9)).all()


def test_scale_invariance_of_codes():
    X, W = _spd_problem(13, 40, out=16)
    H = o.hessian(X)
    U1 = o.factor_u(o.damp(H, lam_rel=0.01)[0])
    U2 = o.factor_u(o.damp(7.25 * H, lam_rel=0.01)[0])
    a = o.gptq_sweep(W, U1, 3, 8, block=16)
    b = o.gptq_sweep(W, U2, 3, 8, block=16)
    assert np.array_equal(a["codes"], b["codes"])


# ---------------------------------------------------------------- golden ---
def _read_golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(None, 1)
            if ";" in v:
                d[k] = np.array([[float(t) for t in row.split()] for row in v.split(";")])
            else:
                d[k] = np.array([float(t) for t in v.split()])
    return d


def test_golden_three_column_example():
    g = _read_golden("worked_3col_2bit.txt")
    w = g["w"][None, :]
    res = o.gptq_sweep(w, o.factor_u(g["H"]), int(g["bits"][0]), int(g["group"][0]))
    assert res["codes"][0].tolist() == g["codes"].astype(int).tolist()
    assert np.allclose(res["What"][0], g["what"], atol=1e-7)
    assert o.objective(w, res["What"], g["H"]) == pytest.approx(g["J"][0], abs=1e-6)


def test_golden_group_example():
    g = _read_golden("worked_group_2bit.txt")
    w = g["w"][None, :]
    res = o.gptq_sweep(w, o.factor_u(g["H"]), int(g["bits"][0]), int(g["group"][0]))
    assert res["codes"][0].tolist() == g["codes"].astype(int).tolist()
    assert np.allclose(res["scales"][0], g["scales"], rtol=1e-6)
    assert res["zeros"][0].tolist() == g["zeros"].tolist()


# ---------------------------------------------------------------- a7 LoRA --
def _lowrank_problem(seed, n=48, r=4, tokens=400, out=10):
    rng = _rng(seed)
    A, _ = np.linalg.qr(rng.standard_normal((tokens, n)))
    V, _ = np.linalg.qr(rng.standard_normal((n, n)))
    sig = np.concatenate([rng.normal(1.0, 0.1, r), 0.05 * np.arange(1, n - r + 1) ** -0.5])
    X = _to_bf16_bits(((A * sig) @ V.T).astype(np.float32))
    W = 0.02 * rng.standard_normal((out, n))
    return X, W


@pytest.mark.parametrize("seed,r,gap", [(30, 4, "wide"), (31, 7, "wide"), (32, 5, "narrow")])
def test_top_eigvecs_span_top_right_singular_subspace(seed, r, gap):
    """[LoRA] method section 2: L = V_r holds the top-r right singular vectors
    of X.  Checked against the SVD of the data matrix itself (not an
    eigendecomposition of H): same projector, Ritz values equal to the r
    largest squared singular values, and the captured energy ||X V||^2 equal
    to their sum (Ky Fan: the maximum over r-dimensional subspaces)."""
    rng = _rng(seed)
    n, tokens = 40, 300
    A, _ = np.linalg.qr(rng.standard_normal((tokens, n)))
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    if gap == "wide":
        sig = np.concatenate([rng.normal(1.0, 0.1, r), 0.05 * np.arange(1, n - r + 1) ** -0.5])
    else:  # power law: sigma_r / sigma_{r+1} about 1.1
        sig = np.arange(1, n + 1) ** -0.5
    X = _to_bf16_bits(((A * sig) @ Q.T).astype(np.float32))
    Xf = o.bf16_bits_to_f64(X)
    H = o.hessian(X)
    V = o.top_eigvecs(H, r)
    _, sv, Vt = np.linalg.svd(Xf, full_matrices=False)
    Vs = Vt[:r].T
    assert np.abs(V.T @ V - np.eye(r)).max() < 1e-12
    g = (sv[r - 1] ** 2 - sv[r] ** 2) / sv[0] ** 2  # relative spectral gap
    assert np.abs(V @ V.T - Vs @ Vs.T).max() < 1e-12 / g
    ritz = np.sort(np.diag(V.T @ H @ V))[::-1]
    assert np.allclose(ritz, sv[:r] ** 2, rtol=1e-10, atol=0)
    assert np.sum((Xf @ V) ** 2) == pytest.approx(np.sum(sv[:r] ** 2), rel=1e-12)
    # and no other r-dimensional subspace captures more energy
    for _ in range(5):
        B, _ = np.linalg.qr(Vs + 0.05 * rng.standard_normal((n, r)))
        assert np.sum((Xf @ B) ** 2) < np.sum((Xf @ V) ** 2)


def test_lora_matches_schur_and_ridge_closed_forms():
    X, W = _lowrank_problem(20)
    H = o.hessian(X)
    res = o.lora(W, H, 4, 3, 0, block=16, lam_rel=1e-4)
    ref = o.lora_schur(W, H, res["L"], res["lam"], 3, 0, block=16)
    assert np.array_equal(res["codes"], ref["codes"])
    sc = np.abs(ref["R_out"]).max()
    assert np.abs(res["R_out"] - ref["R_out"]).max() <= 1e-7 * sc


def test_lora_eig_qr_factor_equals_cholesky_route():
    X, W = _lowrank_problem(21)
    H = o.hessian(X)
    V = o.top_eigvecs(H, 4)
    Ht = o.augmented_hessian(H, V)
    lam = 1e-2 * np.mean(np.diag(H))
    U1 = o.factor_u_eig_qr(Ht, lam)
    U2 = o.factor_u(Ht + lam * np.eye(Ht.shape[0]))
    assert np.abs(U1 - U2).max() <= 1e-8 * np.abs(U2).max()


def test_lora_rank_zero_is_plain_gptq():
    X, W = _lowrank_problem(22)
    H = o.hessian(X)
    res = o.lora(W, H, 0, 3, 8, block=16, lam_rel=1e-3)
    Hl, _ = o.damp(H, lam_rel=1e-3)
    g = o.gptq_sweep(W, o.factor_u(Hl), 3, 8, block=16)
    assert np.array_equal(res["codes"], g["codes"])
    assert res["J"] == pytest.approx(o.objective(W, g["What"], H), rel=1e-9)


def test_lora_basis_invariance_and_improvement():
    X, W = _lowrank_problem(23)
    H = o.hessian(X)
    a = o.lora(W, H, 4, 3, 0, block=16, lam_rel=1e-4)
    O, _ = np.linalg.qr(_rng(5).standard_normal((4, 4)))
    b = o.lora(W, H, 4, 3, 0, block=16, lam_rel=1e-4, V=a["L"] @ O)
    assert np.array_equal(a["codes"], b["codes"])
    LRa = a["R_out"] @ a["L"].T
    LRb = b["R_out"] @ b["L"].T
    assert np.abs(LRa - LRb).max() <= 1e-7 * np.abs(LRa).max()
    # expected (not a theorem): the rank-r correction lowers the layer objective
    Hl, _ = o.damp(H, lam_rel=1e-4)
    g = o.gptq_sweep(W, o.factor_u(Hl), 3, 0, block=16)
    assert a["J"] < o.objective(W, g["What"], H)


def test_lora_objective_is_identity_of_sweep():
    X, W = _lowrank_problem(24)
    H = o.hessian(X)
    a = o.lora(W, H, 4, 3, 0, block=16, lam_rel=1e-4)
    Hl = a["H_aug"] + a["lam"] * np.eye(H.shape[0] + 4)
    Dt = np.hstack([W - a["What"], -a["R_out"]])
    assert np.sum(a["E"] ** 2) == pytest.approx(np.sum((Dt @ Hl) * Dt), rel=1e-8)
    assert a["J"] == pytest.approx(np.sum((Dt @ a["H_aug"]) * Dt), rel=1e-8)

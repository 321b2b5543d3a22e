"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is the oracle's own source with one plausible mistake planted
(a dropped term, a wrong sign or index, a transposed operand, a wrong
rounding).  The mutant module is loaded on the CPU only, never used elsewhere,
and at least one pin must reject it.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle import gptq_ref as o

SRC = open(os.path.join(os.path.dirname(o.__file__), "gptq_ref.py")).read()

MUTANTS = {
    "update_sign": ("W[:, j + 1:upd_end] -= np.outer(e, U[j, j + 1:upd_end])",
                    "W[:, j + 1:upd_end] += np.outer(e, U[j, j + 1:upd_end])"),
    "update_transposed": ("W[:, j + 1:upd_end] -= np.outer(e, U[j, j + 1:upd_end])",
                          "W[:, j + 1:upd_end] -= np.outer(e, U[j + 1:upd_end, j])"),
    "update_off_by_one": ("W[:, j + 1:upd_end] -= np.outer(e, U[j, j + 1:upd_end])",
                          "W[:, j + 2:upd_end] -= np.outer(e, U[j, j + 2:upd_end])"),
    "no_diag_scaling": ("e = (W[:, j] - what) / U[j, j]", "e = (W[:, j] - what)"),
    "dropped_trailing": ("W[:, b1:] -= E[:, b0:b1] @ U[b0:b1, b1:]", "pass"),
    "zero_point_floor": ("np.clip(np.rint(zraw), F32(0), F32(maxq))", "np.clip(np.floor(zraw), F32(0), F32(maxq))"),
    "zero_point_sign": ("x = ((w32 * r).astype(F32) + z)", "x = ((w32 * r).astype(F32) - z)"),
    "grid_without_zero": ("lo = np.minimum(v32.min(axis=-1), F32(0))", "lo = v32.min(axis=-1)"),
    "hessian_shifted": ("H += Xc.T @ Xc", "H += Xc.T @ np.roll(Xc, 1, axis=0)"),
    "factor_transposed": ("return np.triu(C.T)", "return np.triu(C.T).T"),
    "damping_absolute_only": ("lam = float(lam_abs) + float(lam_rel) * float(np.mean(np.diag(H)))",
                              "lam = float(lam_abs) + float(lam_rel)"),
    "static_group_grid": ("s, r, z = fit(W[:, j:j + group], j // group)",
                          "s, r, z = fit(W0[:, j:j + group], j // group)"),
    "bottom_eigvecs": ("idx = np.argsort(lam_)[::-1][:r]", "idx = np.argsort(lam_)[:r]"),
    "eigvecs_rows": ("    return V[:, idx]\n", "    return V[idx, :].T\n"),
    "code_truncated": ("q = np.clip(np.rint(x), F32(0), F32(maxq))", "q = np.clip(np.floor(x), F32(0), F32(maxq))"),
}


def _load(mut):
    old, new = MUTANTS[mut]
    assert SRC.count(old) >= 1, mut
    src = SRC.replace(old, new)
    if mut == "static_group_grid":
        src = src.replace("    W = np.array(W, dtype=np.float64, copy=True)\n    U = np.asarray(U, dtype=np.float64)\n",
                          "    W = np.array(W, dtype=np.float64, copy=True)\n    W0 = W.copy()\n    U = np.asarray(U, dtype=np.float64)\n", 1)
    m = types.ModuleType("oracle_mutant_" + mut)
    exec(compile(src, "<mutant %s>" % mut, "exec"), m.__dict__)
    return m


def _bits(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _pins(m):
    """Run the pins on module m; return the names of those that fail."""
    fails = []
    rng = np.random.default_rng(0)
    n, out = 32, 12
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    X = _bits((rng.standard_normal((128, n)) * np.arange(1, n + 1) ** -0.5) @ Q.T)
    W = 0.02 * rng.standard_normal((out, n))
    W[0, 3] = 0.2
    H = m.hessian(X, chunk=16)
    # exact Hessian
    Xf = o.bf16_bits_to_f64(X)
    if not np.allclose(H, Xf.T @ Xf, rtol=1e-12, atol=0):
        return ["hessian"]
    Hl, lam = m.damp(H, lam_rel=0.01)
    if not math.isclose(lam, 0.01 * np.trace(Xf.T @ Xf) / n, rel_tol=1e-12):
        fails.append("damping")
    try:
        U = m.factor_u(Hl)
        if np.abs(U @ Hl @ U.T - np.eye(n)).max() > 1e-8:
            fails.append("factor")
    except Exception:
        fails.append("factor-raise")
        U = o.factor_u(Hl)
    for group in (0, 8):
        g = m.gptq_sweep(W, U, 3, group, block=8)
        L = o.ql_lower_from_data(X, math.sqrt(lam))
        b = m.babai(W, L, 3, group)
        if not np.array_equal(g["codes"], b["codes"]):
            fails.append("babai")
        D = W - g["What"]
        if np.abs(D - g["E"] @ U).max() > 1e-10:
            fails.append("identity")
        u = m.gptq_sweep(W, U, 3, group)
        if not np.array_equal(u["codes"], g["codes"]):
            fails.append("blocked")
        # round-to-nearest on a scaled identity, by brute force over the grid
        r = m.gptq_sweep(W, m.factor_u(2.0 * np.eye(n)), 3, group, block=8)
        gg = group or n
        for k in range(n // gg):
            s = r["scales"][:, k].astype(np.float64)
            z = r["zeros"][:, k].astype(np.float64)
            lo = np.minimum(W[:, k * gg:(k + 1) * gg].min(1), 0)
            hi = np.maximum(W[:, k * gg:(k + 1) * gg].max(1), 0)
            if not np.allclose(s * 7, hi - lo, rtol=1e-5):
                fails.append("grid-range")
            grid = s[:, None, None] * (np.arange(8)[None, None, :] - z[:, None, None])
            best = np.abs(W[:, k * gg:(k + 1) * gg, None] - grid).argmin(-1)
            if not np.array_equal(r["codes"][:, k * gg:(k + 1) * gg], best):
                fails.append("rtn")
            if (np.abs(-z * s - lo) > 0.5001 * s).any():
                fails.append("grid-zero")
    # L = V_r spans the top-r right singular subspace of X, by the SVD of the data
    V = m.top_eigvecs(H, 3)
    _, _, Vt = np.linalg.svd(Xf, full_matrices=False)
    if V.shape != (n, 3) or np.abs(V @ V.T - Vt[:3].T @ Vt[:3]).max() > 1e-8:
        fails.append("top-subspace")
    # golden group example
    Hg = np.array([[1, 0.5, 0, 0], [0.5, 1, 0, 0], [0, 0, 1, 0], [0, 0, 0, 1.0]])
    wg = np.array([[0.25, 0.10, -0.20, 0.40]])
    rg = m.gptq_sweep(wg, o.factor_u(Hg), 2, 2)
    if rg["codes"][0].tolist() != [3, 1, 0, 3]:
        fails.append("golden")
    # a group whose grid depends on the compensation of earlier columns
    Hc = np.array([[1.0, 0.9], [0.9, 1.0]])
    wc = np.array([[0.07, 0.30]])
    rc = m.gptq_sweep(wc, o.factor_u(Hc), 2, 1)
    Uc = o.factor_u(Hc)
    w1 = 0.30 - (0.07 - float(rc["What"][0, 0])) / Uc[0, 0] * Uc[0, 1]
    if not math.isclose(float(rc["scales"][0, 1]) * 3, max(w1, 0) - min(w1, 0), rel_tol=1e-5):
        fails.append("group-current")
    return fails


def test_unmutated_oracle_passes_all_pins():
    assert _pins(o) == []


@pytest.mark.parametrize("mut", sorted(MUTANTS))
def test_mutant_is_caught(mut):
    try:
        fails = _pins(_load(mut))
    except Exception as e:  # a pin that raises has rejected the mutant
        fails = ["raised %s" % type(e).__name__]
    assert fails, "planted mistake %s was not caught by any pin" % mut

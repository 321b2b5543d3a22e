"""Helpers that compare the GPU library with the oracle (test infrastructure)."""
import numpy as np

from oracle import gptq_ref as o

TIE = 1e-3  # near-tie window on the value being rounded (|frac - 0.5| < TIE)


def np32(t):
    return t.detach().cpu().numpy()


def check_sweep(gpu, W, U, bits, group, block, H, lam, n_q=None, min_agree=0.995, J_tol=5e-3,
                report=None):
    """Codes/zeros/scales/objective of a GPU sweep against the oracle sweep on the same U.

    Raw code agreement must reach min_agree; after the oracle replays the GPU's
    choice at its own near-ties (and only there) every code and zero point must
    agree exactly.  The GPU's objective must match the oracle's (J_tol) and the
    oracle's evaluation of the GPU's own codes (1e-4)."""
    codes = np32(gpu["codes"])
    zeros = np32(gpu["zeros"]).astype(np.float32)
    scales = np32(gpu["scales"])
    raw = o.gptq_sweep(W, U, bits, group, block, n_q=n_q)
    agree = float(np.mean(raw["codes"] == codes))
    rep = o.gptq_sweep(W, U, bits, group, block, n_q=n_q, replay=dict(codes=codes, zeros=zeros), tie_window=TIE)
    bad_codes = int(np.sum(rep["codes"] != codes))
    bad_zeros = int(np.sum(rep["zeros"] != zeros))
    sc_err = float(np.max(np.abs(rep["scales"].astype(np.float64) - scales) / np.abs(rep["scales"])))
    n = codes.shape[1]
    What_gpu = o.dequantize(codes, scales, zeros, group)
    J_eval = o.objective(np.asarray(W)[:, :n], What_gpu, H) if n_q is None else None
    J_ref = o.objective(np.asarray(W)[:, :n], raw["What"], H) if n_q is None else None
    info = dict(agree=agree, bad_codes=bad_codes, bad_zeros=bad_zeros, forced=rep["forced_codes"],
                forced_zeros=rep["forced_zeros"], scale_err=sc_err, J_gpu=gpu.get("J"), J_eval=J_eval, J_ref=J_ref)
    if report is not None:
        report.update(info)
    assert agree >= min_agree, info
    assert bad_codes == 0 and bad_zeros == 0, info
    assert sc_err < 2e-5, info
    if J_eval is not None:
        if gpu.get("J") is not None:
            assert abs(gpu["J"] - J_eval) <= 1e-4 * J_eval, info
        assert abs(J_eval - J_ref) <= J_tol * J_ref, info
    return info


# ---------------------------------------------------------------------------
# Checks that hold at any size (used where the whole oracle would take too
# long): each one tests the GPU's outputs against the definition of the step
# on a sample, in float64.
# ---------------------------------------------------------------------------
U32 = 2.0 ** -24  # unit roundoff of float32


def check_h_block(H_gpu, Xbits, cols, tol=1e-5):
    """The principal sub-block H[cols][:, cols] against the oracle Gram of
    those columns of X (it is the same sum over tokens).  Returns the relative
    Frobenius error."""
    cols = np.asarray(cols)
    Hb = o.hessian(np.ascontiguousarray(Xbits[:, cols]))
    Hg = np.asarray(H_gpu, dtype=np.float64)[np.ix_(cols, cols)]
    err = float(np.linalg.norm(Hg - Hb) / np.linalg.norm(Hb))
    assert err <= tol, err
    return err


def check_u_rows(U, H, lam, rows):
    """U H_lam U^T = I on the sampled rows, to the rounding bound of storing
    U in float32: |U_i H_lam U_j^T - d_ij| <= 4 u (|U_i| H_abs |U_j|^T) + 1e-12.
    U and H are the GPU's (the factor's own input).  Returns the worst ratio
    of the error to its bound."""
    rows = np.asarray(rows)
    Ur = np.asarray(U, dtype=np.float64)[rows]
    Hl = np.asarray(H, dtype=np.float64) + lam * np.eye(H.shape[0])
    M = Ur @ Hl @ Ur.T
    B = 4 * U32 * (np.abs(Ur) @ np.abs(Hl) @ np.abs(Ur).T) + 1e-12
    ratio = float(np.max(np.abs(M - np.eye(len(rows))) / B))
    assert ratio <= 1.0, ratio
    return ratio


def check_sweep_recurrence(W, U, codes, scales, zeros, E, bits, group, n_q=None, tie=TIE):
    """The sweep's defining recurrence on sampled rows, from the GPU's own U
    and errors E (float64 arithmetic):
      v_j = W_j - sum_{i<j} E_i U_ij      (the value the sweep rounds at j)
      grid at a group start from min/max(v of the group's columns, 0)
      q_j = clamp(rne(v_j / s + z))       (either neighbour at a near-tie)
      E_j = (v_j - s (q_j - z)) / U_jj
    Returns a dict of the worst deviations."""
    W = np.asarray(W, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    codes = np.asarray(codes).astype(np.int64)
    scales = np.asarray(scales, dtype=np.float64)
    zeros = np.asarray(zeros).astype(np.int64)
    out, n = codes.shape
    n_q = n if n_q is None else n_q
    maxq = (1 << bits) - 1
    # contributions of all earlier columns: V = W - (E U)_{strictly upper part}
    Us = np.triu(U[:n_q, :n_q], 1)
    V = W[:, :n_q] - E @ Us
    A = np.abs(W[:, :n_q]) + np.abs(E) @ np.abs(Us)  # size of the terms summed into V
    G = group if group else n_q
    worst = dict(code=0, scale=0.0, zero=0, err=0.0)
    for g in range(n_q // G if group else 1):
        j0 = g * G
        if group:
            # the group's columns as they stand when the sweep reaches j0
            vg = W[:, j0:j0 + G] - E[:, :j0] @ U[:j0, j0:j0 + G]
        else:
            vg = W[:, :n_q]
        lo = np.minimum(vg.min(axis=1), 0.0)
        hi = np.maximum(vg.max(axis=1), 0.0)
        s_ref = np.where(hi > lo, (hi - lo) / maxq, 1.0)
        zraw = np.where(hi > lo, -lo / s_ref, 0.0)
        s_g = scales[:, g]
        worst["scale"] = max(worst["scale"], float(np.max(np.abs(s_g - s_ref) / s_ref)))
        z_ok = (zeros[:, g] == np.rint(zraw)) | (np.abs(zraw - np.floor(zraw) - 0.5) < tie)
        worst["zero"] += int(np.sum(~z_ok))
        cols = slice(j0, j0 + G)
        x = V[:, cols] / s_g[:, None] + zeros[:, g][:, None]
        q_ref = np.clip(np.rint(x), 0, maxq)
        near = np.abs(x - np.floor(x) - 0.5) < tie
        neighbour = (codes[:, cols] == np.clip(np.floor(x), 0, maxq)) | (codes[:, cols] == np.clip(np.floor(x) + 1, 0, maxq))
        ok = (codes[:, cols] == q_ref) | (near & neighbour)
        worst["code"] += int(np.sum(~ok))
        what = s_g[:, None] * (codes[:, cols] - zeros[:, g][:, None])
        e_ref = (V[:, cols] - what) / np.diag(U)[cols][None, :]
        scale_e = A[:, cols] / np.diag(U)[cols][None, :] + np.abs(e_ref) + 1e-30
        worst["err"] = max(worst["err"], float(np.max(np.abs(E[:, cols] - e_ref) / scale_e)))
    assert worst["code"] == 0 and worst["zero"] == 0, worst
    assert worst["scale"] < 1e-5, worst
    assert worst["err"] < 1e-4, worst
    return worst

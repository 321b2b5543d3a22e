"""Plain float64 CPU oracle of the GPTQ layer-quantization pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header, table
or constant with the HIP library; it is slow on purpose and written so that
each step can be read against the pages it follows.

Sources (web pages on the subject; each function cites the passage it follows)
  [LoRA] "Technical summary: GPTQ-intrinsic LoRA" (gist.science, 2606.01412)
  [2D]   "GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding" (gist.science,
         2607.27042), technical summary
  [Wiki] "GPTQ" encyclopedia entry (wikiprompt.org)
  [Lat]  "The Lattice Geometry of Neural Network Quantization -- A Short
         Equivalence Proof of GPTQ and Babai's Algorithm" (gist.science,
         2508.01077), technical overview

Conventions.  W is stored as a Linear weight, [out, n] (rows = output neurons,
columns = input dimensions); the pages write XW with W as [n, out].  X is the
calibration matrix [tokens, n]; bfloat16 inputs arrive as their uint16 bit
patterns.  H = X^T X is [n, n].

What pins each function (tests/test_oracle_*.py): exact rational Hessians and
two summation orders; three independent factor routes (Cholesky->inverse->
Cholesky, reversal, QL of the data matrix [X; mu I]); H = cI reduces to
round-to-nearest found by brute force over the grid; the exact identities
W - What = E U and sum(E^2) = tr(D H_lam D^T); blocked == unblocked; GPTQ codes
== an independently written Babai nearest-plane solver on the QL basis; brute
force over all 2-bit code vectors for n <= 8; the nearest-plane error bound;
hand-worked fixtures in tests/golden/; for the LoRA variant the Schur-complement
and ridge (optimal low-rank compensation) closed forms, r = 0 reduction and
basis invariance; for the refinement loop (tests/test_oracle_refine.py) the
truncated SVD at H = I, a matrix-square-root route to the same OLrC optimum,
brute force over the grid for every Bid-Up coordinate decision, the decoupled
(diagonal H) case reducing to round-to-nearest, and a non-increasing trace;
for two-sided rounding (tests/test_oracle_2d.py) the vectorized sweep with the
Kronecker Gram ([2D] Theorem 2), a second topological order (Theorem 1), the
one-sided reductions B = I and A = I, an independently written nearest-plane
solver on the integer lattice, the identity metric and the objective formed
from A and B directly; for the quantised-input target
(tests/test_oracle_qronos.py) the X_q = X reduction to GPTQ, the
completed-square identity over random codes, a least-squares route to the
target, the nearest-plane solver on the target and the objective formed from
the data; for the deployable outputs (tests/test_oracle_deploy.py) the round
trip of packed codes, the nibble and byte layouts at 4 and 8 bits, a
hand-worked 3-bit row, per-vector round-to-nearest of L and R against the
nearest grid level, the dequant GEMM against the dequantised weights, and
the bf16 rounding against torch's float32 -> bfloat16 conversion and
hand-worked ties.  Parity unpinned: the packed layout is a storage convention
of ours.

Parity unpinned (conventions that only self-consistency fixes; the GPU follows
them exactly): the min-max grid details of ``grid_fit`` (0 inside the range,
integer zero point, degenerate range -> s = 1, z = 0) and the moment at which a
group's grid is fitted.

Decision precision.  The pages fix no precision for the rounding decisions, so
they are taken in the library's float32 form x = fl32(fl32(w * fl32(1/s)) + z).
A pin (tests/test_oracle_pins.py) shows that this equals the plain float64
definitions s = (hi - lo)/maxq, z = rne(-lo/s), q = clamp(rne(w/s + z))
everywhere except within the float32 rounding bound of a tie (a few 1e-6),
far inside the 1e-3 near-tie window of the parity protocol.  The top-r
eigenvectors of H are pinned against the SVD of the data matrix.
"""
from __future__ import annotations

import itertools

import numpy as np
import scipy.linalg as sla

F32 = np.float32


class NotPositiveDefinite(ValueError):
    """Raised when the damped Hessian is not positive definite.

    ``info`` follows the library convention: 1 + the index (in H's own
    numbering) of the first pivot found non-positive when columns are
    eliminated from n-1 down to 0.
    """

    def __init__(self, info: int):
        super().__init__(f"damped Hessian not positive definite (info={info})")
        self.info = info


# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) exactly into float64."""
    b = np.ascontiguousarray(np.asarray(bits).astype(np.uint16)).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _as_f64(X) -> np.ndarray:
    X = np.asarray(X)
    if X.dtype == np.uint16 or X.dtype == np.int16:
        return bf16_bits_to_f64(X.view(np.uint16))
    return X.astype(np.float64)


# --------------------------------------------------------------------------
# a1: calibration Hessian
# --------------------------------------------------------------------------
def hessian(X, chunk: int = 2048, H0: np.ndarray | None = None) -> np.ndarray:
    """H = H0 + sum_t x_t^T x_t, unscaled, in float64, streamed over tokens.

    [Lat] tech. overview section 2 (the output error is a sum over the
    calibration samples x_1..x_k) and section 3.1 (the Gram matrix X^T X);
    [2D] section 1 (Gram G = A^T A of the one-sided problem).  bf16 x bf16
    products are exact in float64.
    """
    X = np.asarray(X)
    tokens, n = X.shape
    H = np.zeros((n, n)) if H0 is None else np.array(H0, dtype=np.float64, copy=True)
    for t0 in range(0, tokens, chunk):
        Xc = _as_f64(X[t0:t0 + chunk])
        H += Xc.T @ Xc
    return H


# --------------------------------------------------------------------------
# a2: damping
# --------------------------------------------------------------------------
def damp(H: np.ndarray, lam_abs: float = 0.0, lam_rel: float = 0.0):
    """H_lam = H + lam I with lam = lam_abs + lam_rel * mean(diag H).

    [Lat] section 3.1: stacking mu I under X keeps the lattice basis
    independent and is the same as the lambda-regularisation X^T X + lam I
    (lam = mu^2).  Returns (H_lam, lam).
    """
    n = H.shape[0]
    lam = float(lam_abs) + float(lam_rel) * float(np.mean(np.diag(H)))
    return H + lam * np.eye(n), lam


# --------------------------------------------------------------------------
# a3: upper Cholesky factor of the inverse (three independent routes)
# --------------------------------------------------------------------------
def _chol_lower(A: np.ndarray, reversed_order: bool = False) -> np.ndarray:
    c, info = sla.lapack.dpotrf(np.asarray(A, dtype=np.float64), lower=1, clean=1)
    if info > 0:
        n = A.shape[0]
        # report in H's own numbering, for elimination from n-1 down to 0
        raise NotPositiveDefinite((n - info + 1) if reversed_order else info)
    if info < 0:
        raise ValueError("dpotrf argument error")
    return c


def factor_u(H_lam: np.ndarray) -> np.ndarray:
    """U upper, positive diagonal, with H_lam^{-1} = U^T U.

    Route: Cholesky of H_lam, triangular inverse, explicit inverse Gram,
    Cholesky again.  [2D] sections 2 and 4: the feedback factors are the
    unit-triangular factors of the inverse Gram matrix (its LDL); the unit
    upper one is diag(U)^{-1} U.
    """
    n = H_lam.shape[0]
    _chol_lower(H_lam[::-1, ::-1], reversed_order=True)  # PD check, library numbering
    L = _chol_lower(H_lam)
    Linv = sla.solve_triangular(L, np.eye(n), lower=True)
    Hinv = Linv.T @ Linv
    Hinv = 0.5 * (Hinv + Hinv.T)
    C = _chol_lower(Hinv)
    return np.triu(C.T)


def factor_u_reversal(H_lam: np.ndarray) -> np.ndarray:
    """Same U by the reversal identity U = P chol(P H_lam P)^{-1} P.

    With P the reversal permutation and C = chol(P H_lam P) lower,
    H_lam^{-1} = (P C^{-1} P)^T (P C^{-1} P) and P C^{-1} P is upper with a
    positive diagonal, so it is U (the factor is unique).
    """
    n = H_lam.shape[0]
    C = _chol_lower(H_lam[::-1, ::-1], reversed_order=True)
    Cinv = sla.solve_triangular(C, np.eye(n), lower=True)
    return np.triu(Cinv[::-1, ::-1])


def ql_lower_from_data(X, mu: float) -> np.ndarray:
    """Lower L with L^T L = X^T X + mu^2 I, from a QL factorisation of [X; mu I].

    [Lat] section 3.1 (the stacked basis X' = [X; mu I]) and section 3.3
    (the QL decomposition X = QL links data space and parameter space).
    QL of X' is the QR of X' with its columns reversed, reversed back.
    """
    Xd = _as_f64(X)
    n = Xd.shape[1]
    Xs = np.vstack([Xd, mu * np.eye(n)]) if mu else Xd
    R = np.linalg.qr(Xs[:, ::-1], mode="r")
    L = R[::-1, ::-1].copy()  # lower triangular
    sgn = np.sign(np.diag(L))
    sgn[sgn == 0] = 1.0
    return np.tril(sgn[:, None] * L)


def ql_lower_from_gram(H_lam: np.ndarray) -> np.ndarray:
    """Lower L with L^T L = H_lam from a QL factorisation of a square root of H_lam."""
    lam_, V = np.linalg.eigh(H_lam)
    if np.min(lam_) <= 0:
        raise NotPositiveDefinite(0)
    S = np.sqrt(lam_)[:, None] * V.T  # S^T S = H_lam
    R = np.linalg.qr(S[:, ::-1], mode="r")
    L = R[::-1, ::-1].copy()
    sgn = np.sign(np.diag(L))
    return np.tril(sgn[:, None] * L)


# --------------------------------------------------------------------------
# the asymmetric min-max grid; decisions taken in float32
# --------------------------------------------------------------------------
def grid_fit(v: np.ndarray, maxq: int):
    """Per-row asymmetric min-max grid of 2^b levels over the last axis of v.

    [Wiki] technical approach: weights are split into groups and each group has
    its own scale.  The grid is lo = min(min v, 0), hi = max(max v, 0),
    s = (hi - lo)/maxq, r = 1/s, z = rne(-lo * r) in [0, maxq]; a degenerate
    range (hi == lo) gives s = 1, z = 0.  The zero-point decision is taken in
    float32 (the library's precision).  Returns float32 arrays (s, r, z, zraw)
    where zraw is the value that was rounded to z.
    """
    v32 = np.asarray(v, dtype=np.float64).astype(F32)
    lo = np.minimum(v32.min(axis=-1), F32(0))
    hi = np.maximum(v32.max(axis=-1), F32(0))
    deg = hi == lo
    s = np.where(deg, F32(1), (hi - lo) / F32(maxq)).astype(F32)
    r = (F32(1) / s).astype(F32)
    zraw = ((-lo * r) + F32(0)).astype(F32)  # + 0 turns -0 into +0
    z = np.where(deg, F32(0), np.clip(np.rint(zraw), F32(0), F32(maxq))).astype(F32)
    return s, r, z, zraw


def quantize_values(w: np.ndarray, s, r, z, maxq: int):
    """Round current weights onto the grid (decision in float32).

    x = fl32(fl32(w * r) + z), q = clamp(rne(x), 0, maxq), what = fl32(s (q - z)).
    Returns (q as float32, what as float64, x).
    """
    w32 = np.asarray(w, dtype=np.float64).astype(F32)
    x = ((w32 * r).astype(F32) + z).astype(F32)
    q = np.clip(np.rint(x), F32(0), F32(maxq)).astype(F32)
    what = (s * (q - z)).astype(F32)
    return q, what.astype(np.float64), x


def _near_tie(v, window):
    f = v.astype(np.float64) - np.floor(v.astype(np.float64))
    return np.abs(f - 0.5) < window


# --------------------------------------------------------------------------
# a4/a5: the column sweep, unblocked and with lazy block updates
# --------------------------------------------------------------------------
def gptq_sweep(W, U, bits: int, group: int = 0, block: int | None = None,
               n_q: int | None = None, replay: dict | None = None,
               tie_window: float = 1e-3) -> dict:
    """GPTQ column sweep of W [out, n_total] against U (H_lam^{-1} = U^T U).

    Each row is independent ([Lat] section 2: the problem splits into one
    closest-vector problem per neuron).  For each row, for j = 0..n_q-1 in
    natural order ([2D] section 1: fixed order, error fed forward through a
    triangular feedback matrix; [Wiki] technical approach: quantise a column,
    then update the remaining weights to compensate, in closed form):
      if group and j % group == 0: fit the grid on the current w[j:j+group]
      q_j = clamp(rne(w_j / s + z)),  what_j = s (q_j - z)
        (the decision taken in float32 as fl32(fl32(w_j * fl32(1/s)) + z);
        see the module docstring)
      E_j = (w_j - what_j) / U_jj,    w[k] -= E_j U_jk for k > j
    With ``block`` the update of step j only reaches the columns of its own
    block; after the block, W[:, b1:] -= E[:, b0:b1] U[b0:b1, b1:] ([2D]
    section 2, GPTQ's lazy block update).  ``block=None`` is the unblocked
    sweep.  Columns n_q..n_total-1 are never rounded; they only receive
    updates (the intrinsic-LoRA variant).  group == 0 fits one grid per row on
    the original row.

    ``replay``: dict(codes=..., zeros=...) from another implementation; at a
    near-tie (|frac - 0.5| < tie_window of the value being rounded) where it
    chose the other neighbour, its choice is taken.  Used only by parity tests.
    """
    W = np.array(W, dtype=np.float64, copy=True)
    U = np.asarray(U, dtype=np.float64)
    out, n_total = W.shape
    n_q = n_total if n_q is None else int(n_q)
    maxq = (1 << bits) - 1
    if group:
        assert n_q % group == 0, "group must divide the quantised width"
    B = n_q if block is None else int(block)
    unblocked = block is None
    if group and not unblocked:
        assert group % B == 0 or B % group == 0, "groups must align with blocks"
    ngroups = n_q // group if group else 1
    codes = np.zeros((out, n_q), dtype=np.uint8)
    E = np.zeros((out, n_q))
    What = np.zeros((out, n_q))
    scales = np.zeros((out, ngroups), dtype=F32)
    zeros = np.zeros((out, ngroups), dtype=F32)
    forced_codes = 0
    forced_zeros = 0
    margin = np.full((out, n_q), np.inf)

    def fit(cols, g):
        nonlocal forced_zeros
        s, r, z, zraw = grid_fit(cols, maxq)
        if replay is not None and "zeros" in replay:
            zr = np.asarray(replay["zeros"])[:, g].astype(F32)
            lo = np.clip(np.floor(zraw), 0, maxq).astype(F32)
            hi = np.clip(np.floor(zraw) + 1, 0, maxq).astype(F32)
            take = _near_tie(zraw, tie_window) & (zr != z) & ((zr == lo) | (zr == hi))
            forced_zeros += int(take.sum())
            z = np.where(take, zr, z).astype(F32)
        scales[:, g] = s
        zeros[:, g] = z
        return s, r, z

    if not group:
        s, r, z = fit(W[:, :n_q], 0)
    for b0 in range(0, n_q, B):
        b1 = min(b0 + B, n_q)
        upd_end = n_total if unblocked else b1
        for j in range(b0, b1):
            if group and j % group == 0:
                s, r, z = fit(W[:, j:j + group], j // group)
            q, what, x = quantize_values(W[:, j], s, r, z, maxq)
            margin[:, j] = np.abs((x.astype(np.float64) - np.floor(x.astype(np.float64))) - 0.5)
            if replay is not None and "codes" in replay:
                qr = np.asarray(replay["codes"])[:, j].astype(F32)
                lo = np.clip(np.floor(x), 0, maxq).astype(F32)
                hi = np.clip(np.floor(x) + 1, 0, maxq).astype(F32)
                take = _near_tie(x, tie_window) & (qr != q) & ((qr == lo) | (qr == hi))
                if take.any():
                    forced_codes += int(take.sum())
                    q = np.where(take, qr, q).astype(F32)
                    what = (s * (q - z)).astype(F32).astype(np.float64)
            codes[:, j] = q.astype(np.uint8)
            What[:, j] = what
            e = (W[:, j] - what) / U[j, j]
            E[:, j] = e
            W[:, j + 1:upd_end] -= np.outer(e, U[j, j + 1:upd_end])
        if not unblocked and b1 < n_total:
            W[:, b1:] -= E[:, b0:b1] @ U[b0:b1, b1:]
    return dict(codes=codes, scales=scales, zeros=zeros, E=E, What=What,
                W_final=W, forced_codes=forced_codes, forced_zeros=forced_zeros,
                margin=margin)


def dequantize(codes, scales, zeros, group: int = 0) -> np.ndarray:
    """What = s (q - z) per group, in float32 arithmetic (as stored)."""
    codes = np.asarray(codes).astype(F32)
    out, n = codes.shape
    g = group if group else n
    s = np.repeat(np.asarray(scales, dtype=F32), g, axis=1)[:, :n]
    z = np.repeat(np.asarray(zeros, dtype=F32), g, axis=1)[:, :n]
    return (s * (codes - z)).astype(F32).astype(np.float64)


# --------------------------------------------------------------------------
# a6: objective
# --------------------------------------------------------------------------
def objective(W, What, H) -> float:
    """J = ||X (W - What)^T||_F^2 = tr(D H D^T), D = W - What.

    [LoRA] problem statement (layer-wise reconstruction error) and [Lat]
    section 2 (sum over samples of ||W x_j - V x_j||^2).
    """
    D = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    return float(np.sum((D @ H) * D))


def objective_rows(W, What, H) -> np.ndarray:
    D = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    return np.sum((D @ H) * D, axis=1)


# --------------------------------------------------------------------------
# the whole pass for one layer
# --------------------------------------------------------------------------
def gptq_layer(W, X, bits: int, group: int, block: int, lam_rel: float = 0.01,
               lam_abs: float = 0.0, H: np.ndarray | None = None) -> dict:
    """Hessian -> damping -> factor -> blocked sweep -> objective."""
    if H is None:
        H = hessian(X)
    H_lam, lam = damp(H, lam_abs, lam_rel)
    U = factor_u(H_lam)
    res = gptq_sweep(W, U, bits, group, block)
    res.update(H=H, U=U, lam=lam)
    res["J"] = objective(W, res["What"], H)
    res["J_lam"] = float(np.sum(res["E"] ** 2))
    return res


# --------------------------------------------------------------------------
# independent cross-checks
# --------------------------------------------------------------------------
def babai(W, L, bits: int, group: int = 0) -> dict:
    """Box-constrained Babai nearest-plane on the lattice basis L (H_lam = L^T L).

    [Lat] sections 3.2-3.3 and 4: nearest plane with the (lower) QL factor,
    shown there to take exactly GPTQ's steps.  Coordinate j is rounded at
    c_j = w_j + L[j, :j] (w - v)[:j] / L_jj; for groups the grid is fitted on
    the projected targets u = w[j:] + L[j:, j:]^{-1} L[j:, :j] (w - v)[:j].
    """
    W = np.asarray(W, dtype=np.float64)
    L = np.asarray(L, dtype=np.float64)
    out, n = W.shape
    maxq = (1 << bits) - 1
    V = np.zeros((out, n))
    codes = np.zeros((out, n), dtype=np.uint8)
    ng = n // group if group else 1
    scales = np.zeros((out, ng), dtype=F32)
    zeros = np.zeros((out, ng), dtype=F32)
    if not group:
        s, r, z, _ = grid_fit(W, maxq)
        scales[:, 0], zeros[:, 0] = s, z
    for j in range(n):
        D = W[:, :j] - V[:, :j]
        if group and j % group == 0:
            rhs = L[j:, :j] @ D.T  # [n-j, out]
            u = W[:, j:] + sla.solve_triangular(L[j:, j:], rhs, lower=True).T
            s, r, z, _ = grid_fit(u[:, :group], maxq)
            scales[:, j // group], zeros[:, j // group] = s, z
        c = W[:, j] + (D @ L[j, :j]) / L[j, j]
        q, what, _ = quantize_values(c, s, r, z, maxq)
        codes[:, j] = q.astype(np.uint8)
        V[:, j] = what
    return dict(codes=codes, scales=scales, zeros=zeros, What=V)


def brute_force_row(w, H_lam, s: float, z: float, maxq: int):
    """Exact minimum of (w - what)^T H_lam (w - what) over all code vectors.

    Enumerates every q in {0..maxq}^n (tiny n only) on a fixed grid.
    Returns (min value, argmin codes).
    """
    w = np.asarray(w, dtype=np.float64)
    n = w.shape[0]
    Q = np.array(list(itertools.product(range(maxq + 1), repeat=n)), dtype=np.float64)
    What = (F32(s) * (Q.astype(F32) - F32(z))).astype(F32).astype(np.float64)
    D = w[None, :] - What
    vals = np.einsum("ij,jk,ik->i", D, H_lam, D)
    k = int(np.argmin(vals))
    return float(vals[k]), Q[k].astype(np.uint8)


# --------------------------------------------------------------------------
# a7: GPTQ-intrinsic LoRA
# --------------------------------------------------------------------------
def top_eigvecs(H: np.ndarray, r: int) -> np.ndarray:
    """Eigenvectors of the r largest eigenvalues of H (= top right singular
    vectors of X).  [LoRA] method section 2 (L = V_r)."""
    lam_, V = np.linalg.eigh(H)
    idx = np.argsort(lam_)[::-1][:r]
    return V[:, idx]


def augmented_hessian(H: np.ndarray, V: np.ndarray) -> np.ndarray:
    """H~ = T^T H T with T = [I, V]: the Gram of X~ = [X, X V] without forming X~.

    [LoRA] method section 2 (augmented calibration matrix X~ = [X, XL])."""
    n = H.shape[0]
    T = np.hstack([np.eye(n), V])
    return T.T @ H @ T


def factor_u_eig_qr(Ht: np.ndarray, lam: float) -> np.ndarray:
    """U for the singular augmented Hessian via eigendecomposition and QR.

    [LoRA] method section 2, implementation details: H~ = Q diag(l) Q^T,
    l clamped at 0, S = diag((l + lam)^{-1/2}) Q^T so S^T S = (H~ + lam I)^{-1};
    QR of S gives U = R with rows sign-fixed to a positive diagonal.
    """
    l, Q = np.linalg.eigh(Ht)
    l = np.maximum(l, 0.0)
    S = (1.0 / np.sqrt(l + lam))[:, None] * Q.T
    R = np.linalg.qr(S, mode="r")
    sgn = np.sign(np.diag(R))
    sgn[sgn == 0] = 1.0
    return np.triu(sgn[:, None] * R)


def lora(W, H, r: int, bits: int, group: int = 0, block: int | None = 128,
         lam_rel: float = 1e-4, lam_abs: float = 0.0, V: np.ndarray | None = None,
         replay: dict | None = None) -> dict:
    """GPTQ-intrinsic LoRA: sweep W~ = [W, 0] on the augmented Hessian.

    [LoRA] method section 2: the first n columns are rounded into Q, the r
    appended columns start at zero and absorb the error, giving R.  lam is
    relative to the plain H.  Returns codes/scales/zeros, L = V_r [n, r],
    R [r, out] (pages' convention W^T ~ Q + L R), R_out = R^T, the objective
    J = ||X (W - What - R_out V^T)^T||^2 and J_lam = sum(E^2).
    """
    W = np.asarray(W, dtype=np.float64)
    out, n = W.shape
    lam = float(lam_abs) + float(lam_rel) * float(np.mean(np.diag(H)))
    if V is None:
        V = top_eigvecs(H, r)
    if r == 0:
        V = np.zeros((n, 0))
    Ht = augmented_hessian(H, V)
    U = factor_u_eig_qr(Ht, lam)
    Wt = np.hstack([W, np.zeros((out, r))])
    res = gptq_sweep(Wt, U, bits, group, block, n_q=n, replay=replay)
    Rout = res["W_final"][:, n:]
    D = W - res["What"] - Rout @ V.T
    res.update(L=V, R=Rout.T.copy(), R_out=Rout, U=U, lam=lam, H_aug=Ht)
    res["J"] = float(np.sum((D @ H) * D))
    res["J_lam"] = float(np.sum(res["E"] ** 2))
    return res


def lora_schur(W, H, V, lam: float, bits: int, group: int = 0, block: int | None = 128):
    """Closed forms the LoRA sweep must reproduce.

    Eliminating the r free columns leaves the Schur complement
    S = H_lam - H V (V^T H V + lam I)^{-1} V^T H for the rounded columns, and
    for a fixed Q the optimal compensation is the ridge solution
    R_out^T = (V^T H V + lam I)^{-1} V^T H (W - What)^T ([LoRA] section 4:
    OLrC optimises L, R for a fixed Q).
    """
    n = H.shape[0]
    r = V.shape[1]
    H_lam = H + lam * np.eye(n)
    HV = H @ V
    K = V.T @ HV + lam * np.eye(r)
    S = H_lam - HV @ np.linalg.solve(K, HV.T)
    S = 0.5 * (S + S.T)
    U = factor_u(S)
    res = gptq_sweep(W, U, bits, group, block)
    D1 = np.asarray(W, dtype=np.float64) - res["What"]
    Rt = np.linalg.solve(K, HV.T @ D1.T)
    res.update(R_out=Rt.T, S=S, U=U)
    return res


# --------------------------------------------------------------------------
# refinement after the intrinsic LoRA: OLrC <-> Bid-Up
# --------------------------------------------------------------------------
def olrc(W, What, H, r: int) -> dict:
    """Optimal low-rank compensation for a fixed Q ([LoRA] section 4, OLrC).

    Minimises J(C) = tr((E - C) H (E - C)^T), E = W - What, over rank(C) <= r
    (the layer objective with What + C in place of What).  With any H = F F^T,
    J = ||(E - C) F||_F^2, so by Eckart-Young the best C F is the rank-r
    truncation of E F, P_r P_r^T E F with P_r the top-r left singular vectors
    of E F, i.e. the top-r eigenvectors of E H E^T; hence C = P_r P_r^T E
    (no square root or inverse of H is needed, and a singular H is fine).
    Factors: R_out = P_r [out, r] and L = E^T P_r [n, r], C = R_out L^T
    (the pages' W^T ~ Q + L R with R = R_out^T).  J = tr((E - C) H (E - C)^T).
    """
    W = np.asarray(W, dtype=np.float64)
    E = W - np.asarray(What, dtype=np.float64)
    M = E @ H @ E.T
    lam_, P = np.linalg.eigh(M)
    P = P[:, np.argsort(lam_)[::-1][:r]]
    L = E.T @ P
    C = P @ L.T
    D = E - C
    return dict(R_out=P, L=L, C=C, J=float(np.sum((D @ H) * D)), eig=np.sort(lam_)[::-1])


def bid_up(W, C, codes, scales, zeros, H, bits: int, group: int = 0,
           replay=None, tie_window: float = 1e-3) -> dict:
    """One Bid-Up pass: coordinate moves of Q on its fixed grid for fixed L, R.

    [LoRA] section 4, Bid-Up: with the low-rank part C = R_out L^T fixed and
    the grid (scales, zeros) fixed, each row's objective
    J_i(q) = d H d^T, d = w - c - what(q), is lowered one coordinate at a
    time.  Along coordinate j, J_i is a parabola in what_j with its vertex at
    t = what_j + g_j / H_jj, g = d H (the gradient is -2 g), so the best grid
    value is the one nearest t: q* = clamp(rne(x)), x = fl32(fl32(t r) + z)
    (the sweep's rounding, in float32); the code moves to q* only when that
    strictly lowers J_i, |x - q*| < |x - q_j|, and the move delta = what(q*)
    - what(q_j) changes d_j by -delta and g by -delta H_j:.  Coordinates are
    visited once, j = 0..n-1 (plain reading: one cyclic pass per Bid-Up step).

    ``replay``: codes from another implementation of the same pass; where x
    is within tie_window of the midpoint between its choice and ours (the
    choices differ by one level), its choice is taken.  Returns the new codes,
    What, the per-move objective changes and J before and after.
    """
    W = np.asarray(W, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    out, n = W.shape
    maxq = (1 << bits) - 1
    codes = np.array(codes, dtype=np.uint8, copy=True)
    What = dequantize(codes, scales, zeros, group)
    g = (W - np.asarray(C, dtype=np.float64) - What) @ H
    J0 = float(np.sum(g * (W - C - What)))
    gs = group if group else n
    dJ = np.zeros(out)
    moves = 0
    forced = 0
    for j in range(n):
        s = np.asarray(scales, dtype=F32)[:, j // gs]
        z = np.asarray(zeros, dtype=F32)[:, j // gs]
        rr = (F32(1) / s).astype(F32)
        qo = codes[:, j].astype(F32)
        ho = What[:, j]
        t = (ho + g[:, j] / H[j, j]).astype(F32)
        x = ((t * rr).astype(F32) + z).astype(F32)
        qs = np.clip(np.rint(x), F32(0), F32(maxq)).astype(F32)
        mv = np.abs(x - qs) < np.abs(x - qo)
        qn = np.where(mv, qs, qo).astype(F32)
        if replay is not None:
            qr = np.asarray(replay)[:, j].astype(F32)
            mid = F32(0.5) * (qr + qn)
            take = (qr != qn) & (np.abs(qr - qn) == 1) & (np.abs(x.astype(np.float64) - mid) < tie_window)
            forced += int(take.sum())
            qn = np.where(take, qr, qn).astype(F32)
        hn = (s * (qn - z)).astype(F32).astype(np.float64)
        delta = hn - ho
        moves += int(np.count_nonzero(delta))
        dJ += delta * (delta * H[j, j] - 2.0 * g[:, j])
        codes[:, j] = qn.astype(np.uint8)
        What[:, j] = hn
        mv_rows = delta != 0  # rows that did not move keep their g
        g[mv_rows] -= np.outer(delta[mv_rows], H[j])
    D = W - C - What
    return dict(codes=codes, What=What, dJ=dJ, J0=J0, J=float(np.sum((D @ H) * D)),
                moves=moves, forced=forced)


def lora_refine(W, H, r: int, bits: int, group: int = 0, block: int | None = 128,
                lam_rel: float = 1e-4, lam_abs: float = 0.0, rounds: int = 1,
                replay: list | None = None) -> dict:
    """Intrinsic LoRA, then ``rounds`` of OLrC followed by Bid-Up, then a last
    OLrC so that L, R are optimal for the final Q ([LoRA] section 4: the two
    steps alternate; each minimises the objective over its own variables, so
    the objective never increases).  trace = [J after the sweep, then J after
    every step] (2 rounds + 2 values).  ``replay[t]``: codes of another
    implementation after Bid-Up pass t.
    """
    res = lora(W, H, r, bits, group, block, lam_rel=lam_rel, lam_abs=lam_abs)
    codes, What = res["codes"], res["What"]
    trace = [res["J"]]
    steps = []
    for t in range(rounds):
        oc = olrc(W, What, H, r)
        trace.append(oc["J"])
        bu = bid_up(W, oc["C"], codes, res["scales"], res["zeros"], H, bits, group,
                    replay=None if replay is None else replay[t])
        codes, What = bu["codes"], bu["What"]
        trace.append(bu["J"])
        steps.append(dict(olrc=oc, bid_up=bu))
    if rounds:
        oc = olrc(W, What, H, r)
        trace.append(oc["J"])
        L, R_out = oc["L"], oc["R_out"]
    else:
        L, R_out = res["L"], res["R_out"]
    return dict(codes=codes, scales=res["scales"], zeros=res["zeros"], What=What, L=L,
                R=R_out.T.copy(), R_out=R_out, trace=trace, steps=steps, sweep=res)


# --------------------------------------------------------------------------
# GPTQ-2D: two-sided adaptive rounding
# --------------------------------------------------------------------------
def round_1d(x, U, qmin: int, qmax: int, replay=None, tie_window: float = 1e-3) -> dict:
    """One-sided adaptive rounding of a vector to integers ([2D] section 1:
    fixed order, rounding error fed forward through a triangular feedback
    matrix).  U upper with K^{-1} = U^T U for the metric K.  For p in order:
    z_p = clamp(rne(fl32(w_p)), qmin, qmax), e_p = (w_p - z_p) / U_pp,
    w[q] -= e_p U_pq for q > p.  sum(e^2) = (x - z)^T K (x - z).
    ``replay``: integers of another implementation, taken at near-ties.
    """
    w = np.array(x, dtype=np.float64, copy=True).ravel()
    U = np.asarray(U, dtype=np.float64)
    N = w.size
    z = np.zeros(N)
    e = np.zeros(N)
    forced = 0
    for p in range(N):
        v = F32(w[p])
        q = float(np.clip(np.rint(v), qmin, qmax))
        if replay is not None:
            qr = float(np.asarray(replay).ravel()[p])
            if qr != q and abs(qr - q) == 1 and abs(abs(float(v) - min(qr, q)) - 0.5) < tie_window:
                q = qr
                forced += 1
        z[p] = q
        e[p] = (w[p] - q) / U[p, p]
        w[p + 1:] -= e[p] * U[p, p + 1:]
    return dict(z=z, e=e, J=float(np.sum(e * e)), forced=forced)


def round_2d_vectorized(X, UG, UH, qmin: int, qmax: int) -> dict:
    """Two-sided rounding as the 1D sweep on vec(X) ([2D] section 1):
    ||A (Z - X) B||_F^2 = ||(B^T kron A)(vec Z - vec X)||^2 has the Gram
    H kron G (H = B B^T, G = A^T A), and with G^{-1} = UG^T UG,
    H^{-1} = UH^T UH the feedback factor of (H kron G)^{-1} is UH kron UG.
    vec stacks columns, so the order is column-major.  O(m^2 n^2): the
    reference definition, small sizes only.
    """
    X = np.asarray(X, dtype=np.float64)
    m, n = X.shape
    UK = np.kron(np.asarray(UH, dtype=np.float64), np.asarray(UG, dtype=np.float64))
    r = round_1d(X.T.ravel(), UK, qmin, qmax)
    return dict(Z=r["z"].reshape(n, m).T, E=r["e"].reshape(n, m).T, J=r["J"])


def round_2d(X, UG, UH, qmin: int, qmax: int, replay=None, tie_window: float = 1e-3) -> dict:
    """GPTQ-2D: the same rounding trajectory in anti-diagonal stages with lazy
    buffers, O(mn max(m, n)) ([2D] section 2: Kronecker feedback, rank-1
    updates on the lower-right rectangle, anti-diagonal independence, the
    buffer C = L E pushed down columns and then to the right along rows).

    Unit factors: Lg[k, i] = UG[i, k] / UG[i, i] (lower), Uh[j, l] = UH[j, l]
    / UH[j, j] (upper).  Rounding entry (i, j) with delta = w_ij - z_ij
    changes w_kl by -Lg[k, i] delta Uh[j, l] for k >= i, l >= j.  Entry (k, l)
    is reached after every (i, j) with i <= k, j <= l, so its value is
    x_kl - R_kl - C_kl with
      C_kl = sum_{i<k} Lg[k, i] delta_il            (pushed down column l)
      R_kl = sum_{j<l} Cfin_kj Uh[j, l],  Cfin_kj = C_kj + delta_kj
                                                    (pushed right along row k).
    Entries on one anti-diagonal k + l = s touch disjoint columns of C and
    disjoint rows of R, so a stage is parallel.
    """
    X = np.asarray(X, dtype=np.float64)
    UG = np.asarray(UG, dtype=np.float64)
    UH = np.asarray(UH, dtype=np.float64)
    m, n = X.shape
    Lg = (UG / np.diag(UG)[:, None]).T
    Uh = UH / np.diag(UH)[:, None]
    C = np.zeros((m, n))
    R = np.zeros((m, n))
    Z = np.zeros((m, n))
    D = np.zeros((m, n))
    forced = 0
    for s in range(m + n - 1):
        for k in range(max(0, s - n + 1), min(m, s + 1)):
            l = s - k
            w = X[k, l] - R[k, l] - C[k, l]
            v = F32(w)
            q = float(np.clip(np.rint(v), qmin, qmax))
            if replay is not None:
                qr = float(np.asarray(replay)[k, l])
                if qr != q and abs(qr - q) == 1 and abs(abs(float(v) - min(qr, q)) - 0.5) < tie_window:
                    q = qr
                    forced += 1
            d = w - q
            Z[k, l] = q
            D[k, l] = d
            C[k + 1:, l] += Lg[k + 1:, k] * d
            cfin = C[k, l] + d
            R[k, l + 1:] += cfin * Uh[l, l + 1:]
    E = D / np.outer(np.diag(UG), np.diag(UH))
    return dict(Z=Z, E=E, delta=D, J=float(np.sum(E * E)), forced=forced)


def objective_2d(X, Z, G, H) -> float:
    """||A (Z - X) B||_F^2 = tr((Z - X)^T G (Z - X) H) for G = A^T A, H = B B^T."""
    D = np.asarray(Z, dtype=np.float64) - np.asarray(X, dtype=np.float64)
    return float(np.sum((G @ D @ H) * D))


# --------------------------------------------------------------------------
# quantised-input calibration target (Qronos-style)
# --------------------------------------------------------------------------
def cross_gram(Xa, Xb, chunk: int = 2048) -> np.ndarray:
    """Xa^T Xb in float64 (bf16 bit patterns or floats), summed over token
    chunks in order; the two-input form of ``hessian``."""
    A = _as_f64(Xa)
    B = _as_f64(Xb)
    n = A.shape[1]
    G = np.zeros((n, B.shape[1]))
    for t0 in range(0, A.shape[0], chunk):
        G += A[t0:t0 + chunk].T @ B[t0:t0 + chunk]
    return G


def qronos_target(W, Hq, G, lam: float) -> np.ndarray:
    """Target rows w* = (Hq + lam I)^{-1} (G + lam I) w.

    [Lat] section 5.1: when the layer's inputs come from already-quantised
    layers (Xq instead of X), only the target changes.  For every row,
    ||Xq q - X w||^2 + lam ||q - w||^2 = (q - w*)^T (Hq + lam I) (q - w*) +
    const with Hq = Xq^T Xq and G = Xq^T X, so the sweep runs on w* with the
    factor of Hq + lam I.  Damping is a ridge towards w (our reading); with
    Xq = X the target is w itself.
    """
    n = Hq.shape[0]
    Hl = Hq + lam * np.eye(n)
    return np.linalg.solve(Hl, (G + lam * np.eye(n)) @ np.asarray(W, dtype=np.float64).T).T


def gptq_qronos(W, X, Xq, bits: int, group: int, block: int, lam_rel: float = 0.01,
                lam_abs: float = 0.0, replay: dict | None = None) -> dict:
    """GPTQ with the quantised-input target: Hq = Xq^T Xq, G = Xq^T X,
    lam from Hq, W* = qronos_target, U = factor of Hq + lam I, then the sweep
    on W*.  Returns the sweep's result plus W_target, lam, J (the surrogate,
    tr((W* - What) Hq (W* - What)^T)) and J_q = ||Xq What^T - X W^T||_F^2."""
    Hq = hessian(Xq)
    G = cross_gram(Xq, X)
    H = hessian(X)
    Hl, lam = damp(Hq, lam_abs, lam_rel)
    Wst = qronos_target(W, Hq, G, lam)
    U = factor_u(Hl)
    res = gptq_sweep(Wst, U, bits, group, block, replay=replay)
    Q = res["What"]
    Wd = np.asarray(W, dtype=np.float64)
    J_q = float(np.sum((Q @ Hq) * Q) - 2.0 * np.sum((Q @ G) * Wd) + np.sum((Wd @ H) * Wd))
    res.update(W_target=Wst, U=U, lam=lam, Hq=Hq, G=G, J=objective(Wst, Q, Hq), J_q=J_q)
    return res


# --------------------------------------------------------------------------
# deployable outputs: packed codes, low-precision L and R, the dequant GEMM
# --------------------------------------------------------------------------
def pack_codes(codes, bits: int) -> np.ndarray:
    """Rows of codes as little-endian bitstreams in uint32 words: code k of a
    row occupies bits [k bits, (k + 1) bits) of the row's stream (bit b in
    word b // 32 at position b % 32); the row is padded to whole words with
    zero bits.  (A storage convention: the pages give no format.)"""
    codes = np.asarray(codes, dtype=np.int64)
    out, n = codes.shape
    words = (n * bits + 31) // 32
    packed = np.zeros((out, words), dtype=np.uint32)
    for i in range(out):
        stream = 0
        for k in range(n):
            stream |= int(codes[i, k]) << (k * bits)
        for w in range(words):
            packed[i, w] = (stream >> (32 * w)) & 0xFFFFFFFF
    return packed


def unpack_codes(packed, n: int, bits: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint64)
    out = packed.shape[0]
    codes = np.zeros((out, n), dtype=np.uint8)
    for i in range(out):
        stream = 0
        for w in range(packed.shape[1]):
            stream |= int(packed[i, w]) << (32 * w)
        for k in range(n):
            codes[i, k] = (stream >> (k * bits)) & ((1 << bits) - 1)
    return codes


def quantize_lowrank(L, R, bits: int, bits_R: int | None = None) -> dict:
    """Round-to-nearest of the low-rank factors on their own grids ([LoRA]
    results: L and R themselves at low precision, 4 and 8 bits; L at `bits`,
    R at `bits_R`, by default the same): each rank component - a column of L
    [n, r], a row of R [r, out] - gets the min-max grid of ``grid_fit`` and the
    rounding of ``quantize_values`` (decisions in fp32).
    Returns codes, scales, zeros and the dequantised L, R."""
    Lt = np.asarray(L, dtype=np.float64).T  # [r, n]: one component per row
    R = np.asarray(R, dtype=np.float64)
    res = {}
    for name, M, b in (("L", Lt, bits), ("R", R, bits if bits_R is None else bits_R)):
        maxq = (1 << b) - 1
        s, rr, z, _ = grid_fit(M, maxq)
        q, what, _ = quantize_values(M, s[:, None], rr[:, None], z[:, None], maxq)
        res[name + "_codes"] = q.astype(np.uint8)
        res[name + "_scales"] = s
        res[name + "_zeros"] = z
        res[name + "_hat"] = what
    res["L_codes"] = res["L_codes"].T.copy()  # back to [n, r]
    res["L_hat"] = res["L_hat"].T.copy()
    return res


def bf16_round(v) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), returned
    as float32: keep the upper 16 bits of the binary32 pattern after adding
    0x7FFF plus the lowest kept bit (finite inputs)."""
    u = np.asarray(v, dtype=F32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(F32)


def gemm_w4a16(X, codes, scales, zeros, group: int = 0, weight_bf16: bool = False) -> np.ndarray:
    """Y = X What^T in float64 with What = s (q - z) per group as stored
    (``dequantize``): the product a deployed 4-bit layer computes on bf16
    activations (X as bf16 bit patterns or floats).  With weight_bf16 the
    dequantised weights are first rounded to bf16 (``bf16_round``), the
    operand a matrix unit that multiplies bf16 by bf16 is given (our reading:
    the pages fix no arithmetic for the product)."""
    What = dequantize(codes, scales, zeros, group)
    if weight_bf16:
        What = bf16_round(What.astype(F32)).astype(np.float64)
    return _as_f64(X) @ What.T

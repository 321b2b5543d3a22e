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
        assert abs(gpu["J"] - J_eval) <= 1e-4 * J_eval, info
        assert abs(J_eval - J_ref) <= J_tol * J_ref, info
    return info

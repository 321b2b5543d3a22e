"""GPU GPTQ with the quantised-input target against the oracle, through the C ABI.

The target W* = W (G + lam I)^T (Hq + lam I)^{-1} is compared with the
oracle's (float64 Grams) to a bound derived from the fp32 Grams; the sweep is
then checked on the GPU's own target with the oracle's factor (codes exact
after the replay at near-ties), and the true objective ||Xq What^T - X W^T||^2
of the GPU's codes against the oracle pipeline's.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gptq_ref as o  # noqa: E402
from post_weight_quantization_gptq_amd import Context, GPTQError, synth  # noqa: E402
from parity import check_sweep, np32  # noqa: E402

pytestmark = pytest.mark.gpu

SPEC = synth.LayerSpec("qronos", 160, 384, 8192, 4, 128, 128, 0.01, decay=0.4, outlier_channels=4, seed=81)


@pytest.fixture(scope="module")
def ctx():
    c = Context("cuda:0")
    yield c
    c.close()


def _j_q(W, What, Hq, G, H):
    return float(np.sum((What @ Hq) * What) - 2.0 * np.sum((What @ G) * W) + np.sum((W @ H) * W))


@pytest.mark.parametrize("group,block", [(0, 128), (128, 128), (64, 32)])
def test_qronos_matches_oracle(ctx, group, block):
    spec = dataclasses.replace(SPEC, group=group, block=block)
    print("qronos", group, block, flush=True)
    lay = synth.layer(spec)
    Xq = synth.perturbed(lay["X"], spec.seed)
    res = ctx.quantize_qronos(lay["W"].cuda(), lay["X"].cuda(), Xq.cuda(), spec.bits, group, block,
                              lam_rel=spec.lam_rel, want_target=True)
    W = lay["W"].numpy().astype(np.float64)
    Xb, Xqb = synth.bits_to_numpy(lay["X"]), synth.bits_to_numpy(Xq)
    Hq, G, H = o.hessian(Xqb), o.cross_gram(Xqb, Xb), o.hessian(Xb)
    Hl, lam = o.damp(Hq, lam_rel=spec.lam_rel)
    Wst = o.qronos_target(W, Hq, G, lam)
    Wt = np32(res["Wt"]).astype(np.float64)
    # bound: fp32 Grams (relative error ~3e-7) amplified by the condition
    # number of Hq_lam, plus the fp32 storage of W*
    kappa = np.linalg.cond(Hl)
    t_err = float(np.abs(Wt - Wst).max() / np.abs(Wst).max())
    print(dict(kappa=kappa, target_err=t_err), flush=True)
    assert t_err <= 1e-6 * kappa + 1e-6
    rep = {}
    check_sweep(res, Wt, o.factor_u(Hl), spec.bits, group, block, Hq, lam, report=rep)
    ref = o.gptq_qronos(W, Xb, Xqb, spec.bits, group, block, lam_rel=spec.lam_rel)
    What = o.dequantize(np32(res["codes"]), np32(res["scales"]), np32(res["zeros"]).astype(np.float32), group)
    jq = _j_q(W, What, Hq, G, H)
    # plain GPTQ calibrated on the quantised inputs, for comparison (expected
    # to be worse on the true objective, not a theorem)
    plain = o.gptq_layer(W, Xqb, spec.bits, group, block, lam_rel=spec.lam_rel)
    jq_plain = _j_q(W, plain["What"], Hq, G, H)
    print(dict(rep, J_q=jq, J_q_ref=ref["J_q"], J_q_plain_gptq=jq_plain), flush=True)
    assert abs(jq - ref["J_q"]) <= 5e-3 * ref["J_q"]
    assert jq < jq_plain


def test_same_inputs_give_gptq(ctx):
    spec = SPEC
    lay = synth.layer(spec)
    X = lay["X"].cuda()
    res = ctx.quantize_qronos(lay["W"].cuda(), X, X, spec.bits, spec.group, spec.block, lam_rel=spec.lam_rel,
                              want_target=True)
    H = ctx.hessian(X)
    U, _, lam = ctx.factor(H, lam_rel=spec.lam_rel)
    g = ctx.quantize(lay["W"].cuda(), U, spec.bits, spec.group, spec.block, lam)
    W = lay["W"].numpy().astype(np.float64)
    t_err = float(np.abs(np32(res["Wt"]) - W).max() / np.abs(W).max())
    agree = float(np.mean(np32(res["codes"]) == np32(g["codes"])))
    print(dict(target_err=t_err, agree=agree), flush=True)
    assert t_err <= 1e-4
    assert agree >= 0.999


def test_qronos_rejects_unsupported_shapes(ctx):
    W = torch.zeros((8, 40), device="cuda")
    X = torch.zeros((64, 40), dtype=torch.int16, device="cuda")
    with pytest.raises(GPTQError):
        ctx.quantize_qronos(W, X, X, 4, 0, 16)

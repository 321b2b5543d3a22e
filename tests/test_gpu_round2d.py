"""GPU two-sided rounding (GPTQ-2D) against the oracle, through the C ABI.

The oracle runs the anti-diagonal algorithm on the same factors the GPU uses
(the GPU's fp32 UG, UH taken as float64), so the comparison isolates the
rounding.  Decisions are fp32 on both sides; where the rounded value sits
within TIE of a midpoint the oracle takes the GPU's choice, and every other
integer must agree exactly.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gptq_ref as o  # noqa: E402
from post_weight_quantization_gptq_amd import Context, GPTQError  # noqa: E402
from parity import TIE, np32  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = Context("cuda:0")
    yield c
    c.close()


def _gram(k, seed, decay=0.5, tokens=None):
    """Gram of a seeded [tokens, k] matrix with an i^-decay spectrum and a Haar rotation."""
    r = np.random.default_rng(seed)
    tokens = tokens or 4 * k
    Q, _ = np.linalg.qr(r.standard_normal((k, k)))
    Y = (r.standard_normal((tokens, k)) * np.arange(1, k + 1) ** -decay) @ Q.T
    return (Y.T @ Y).astype(np.float32)


def _factors(ctx, G, H, lam_rel=0.01):
    UG, _, lg = ctx.factor(torch.from_numpy(G).cuda(), lam_rel=lam_rel)
    UH, _, lh = ctx.factor(torch.from_numpy(H).cuda(), lam_rel=lam_rel)
    return UG, UH, lg, lh


CASES = [(64, 64, -8, 7), (100, 37, -8, 7), (130, 200, -8, 7), (1, 70, -8, 7), (70, 1, -8, 7),
         (257, 129, 0, 3), (200, 200, -2, 1)]


@pytest.mark.parametrize("m,n,qmin,qmax", CASES, ids=lambda v: str(v))
def test_round_2d_matches_oracle(ctx, m, n, qmin, qmax):
    print("round_2d", m, n, qmin, qmax, flush=True)
    G, H = _gram(m, m + 1), _gram(n, n + 2)
    UG, UH, lg, lh = _factors(ctx, G, H)
    X = np.random.default_rng(m * 7 + n).normal(0.0, 3.0, (m, n)).astype(np.float32)
    res = ctx.round_2d(torch.from_numpy(X).cuda(), UG, UH, qmin, qmax, want_delta=True)
    Z = np32(res["Z"]).astype(np.float64)
    ug, uh = np32(UG).astype(np.float64), np32(UH).astype(np.float64)
    raw = o.round_2d(X, ug, uh, qmin, qmax)
    rep = o.round_2d(X, ug, uh, qmin, qmax, replay=Z, tie_window=TIE)
    info = dict(agree=float(np.mean(raw["Z"] == Z)), forced=rep["forced"], bad=int(np.sum(rep["Z"] != Z)),
                J=res["J"], J_ref=rep["J"])
    print(info, flush=True)
    assert info["bad"] == 0, info
    assert rep["forced"] <= max(2, 1e-3 * Z.size), info
    assert Z.min() >= qmin and Z.max() <= qmax
    assert abs(res["J"] - rep["J"]) <= 1e-4 * rep["J"], info
    d = np32(res["delta"]).astype(np.float64)
    assert np.abs(d - rep["delta"]).max() <= 1e-3
    # the objective is the two-sided metric of the damped Grams the factors belong to
    Gl = G.astype(np.float64) + lg * np.eye(m)
    Hl = H.astype(np.float64) + lh * np.eye(n)
    assert res["J"] == pytest.approx(o.objective_2d(X, Z, Gl, Hl), rel=1e-3)


def test_identity_factors_round_to_nearest(ctx):
    X = np.random.default_rng(3).normal(0, 4, (90, 70)).astype(np.float32)
    res = ctx.round_2d(torch.from_numpy(X).cuda(), torch.eye(90, device="cuda"), torch.eye(70, device="cuda"), -8, 7)
    assert np.array_equal(np32(res["Z"]), np.clip(np.rint(X), -8, 7).astype(np.int32))


def test_one_sided_case_is_columnwise_rounding(ctx):
    # B = I: each column against G alone ([2D] section 5)
    m, n = 96, 20
    G = _gram(m, 5)
    UG, _, _ = ctx.factor(torch.from_numpy(G).cuda(), lam_rel=0.01)
    X = np.random.default_rng(6).normal(0, 3, (m, n)).astype(np.float32)
    res = ctx.round_2d(torch.from_numpy(X).cuda(), UG, torch.eye(n, device="cuda"), -8, 7)
    Z = np32(res["Z"])
    ug = np32(UG).astype(np.float64)
    for j in range(n):
        r = o.round_1d(X[:, j], ug, -8, 7, replay=Z[:, j], tie_window=TIE)
        assert np.array_equal(r["z"], Z[:, j]), j


def test_round_2d_rejects_bad_arguments(ctx):
    X = torch.zeros((4, 4), device="cuda")
    with pytest.raises(GPTQError):
        ctx.round_2d(X, torch.eye(4, device="cuda"), torch.eye(4, device="cuda"), 3, 2)

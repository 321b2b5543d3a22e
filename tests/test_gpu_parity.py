"""GPU library vs the CPU oracle, element by element, on seeded synthetic layers.

Every test here calls the HIP library through its C ABI (the ctypes binding);
expected values come only from the oracle.  Sizes are small enough for the
oracle to finish in seconds but span several tiles and ragged tails.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gptq_ref as o  # noqa: E402
from post_weight_quantization_gptq_amd import Context, GPTQError, synth  # noqa: E402
from parity import check_sweep, np32  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = Context("cuda:0")
    yield c
    c.close()


def _bits(X):
    return synth.bits_to_numpy(X)


def _rand_x(tokens, n, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((tokens, n), generator=g) * scale
    return x.to(torch.bfloat16).view(torch.int16)


# ------------------------------------------------------------------ Hessian --
@pytest.mark.parametrize("tokens,n", [(1024, 512), (3001, 520), (700, 37), (64, 256), (5000, 1000), (0, 64)])
def test_hessian_matches_oracle(ctx, tokens, n):
    print("hessian", tokens, n, flush=True)
    X = _rand_x(tokens, n, 7 + n)
    H = ctx.hessian(X.cuda())
    torch.cuda.synchronize()
    Hg = np32(H).astype(np.float64)
    Hr = o.hessian(_bits(X))
    den = max(np.linalg.norm(Hr), 1e-30)
    assert np.linalg.norm(Hg - Hr) / den <= 1e-5 or tokens == 0
    if tokens == 0:
        assert np.all(Hg == 0)
    assert np.array_equal(Hg, Hg.T)  # exactly symmetric


def test_hessian_accumulate_and_ld(ctx):
    X = _rand_x(2000, 300, 3)
    Xpad = torch.zeros((2000, 304), dtype=torch.int16)
    Xpad[:, :300] = X
    H = ctx.hessian(Xpad[:1200].cuda(), n=300)
    ctx.hessian(Xpad[1200:].cuda(), n=300, H=H, accumulate=True)
    torch.cuda.synchronize()
    Hr = o.hessian(_bits(X))
    assert np.linalg.norm(np32(H) - Hr) / np.linalg.norm(Hr) <= 1e-5


def test_hessian_bitwise_repeatable(ctx):
    X = _rand_x(4096, 700, 5).cuda()
    a = ctx.hessian(X).clone()
    b = ctx.hessian(X).clone()
    assert torch.equal(a, b)


def test_hessian_unaligned_rows(ctx):
    X = _rand_x(999, 30, 1)  # ldx = 30: rows not 16-byte aligned
    Xpad = torch.zeros((999, 37), dtype=torch.int16)
    Xpad[:, :30] = X
    H = ctx.hessian(X.cuda())
    H2 = ctx.hessian(Xpad.cuda(), n=30)
    torch.cuda.synchronize()
    Hr = o.hessian(_bits(X))
    assert np.linalg.norm(np32(H) - Hr) / np.linalg.norm(Hr) <= 1e-5
    assert torch.equal(H, H2)


# ------------------------------------------------------------------- factor --
def _spd(n, seed, decay=0.8, tokens=None):
    X = _rand_x(tokens or 3 * n, n, seed)
    Xf = o.bf16_bits_to_f64(_bits(X)) * (np.arange(1, n + 1) ** (-decay / 2))
    return Xf.T @ Xf


@pytest.mark.parametrize("n", [64, 100, 200, 517, 1024, 2560])
def test_factor_matches_oracle(ctx, n):
    print("factor", n, flush=True)
    H32 = _spd(n, n).astype(np.float32)
    U, info, lam = ctx.factor(torch.from_numpy(H32).cuda(), lam_rel=0.01)
    torch.cuda.synchronize()
    H64 = H32.astype(np.float64)
    Hl, lam_r = o.damp(H64, lam_rel=0.01)
    Ur = o.factor_u_reversal(Hl)
    assert info == 0
    assert lam == pytest.approx(lam_r, rel=1e-12)
    Ug = np32(U).astype(np.float64)
    assert np.all(np.tril(Ug, -1) == 0)
    assert np.abs(Ug - Ur).max() <= 2e-6 * np.abs(Ur).max()
    assert np.abs(Ug @ Hl @ Ug.T - np.eye(n)).max() < 1e-4


def test_factor_not_pd_reports_pivot(ctx):
    n = 150
    H = np.eye(n, dtype=np.float32)
    H[37, 37] = -1.0
    with pytest.raises(GPTQError) as e:
        ctx.factor(torch.from_numpy(H).cuda(), lam_rel=0.0)
    assert e.value.status == 2
    with pytest.raises(o.NotPositiveDefinite) as r:
        o.factor_u(H.astype(np.float64))
    assert e.value.info == r.value.info == 38


def test_factor_nonfinite(ctx):
    H = np.eye(70, dtype=np.float32)
    H[3, 5] = H[5, 3] = np.nan
    with pytest.raises(GPTQError) as e:
        ctx.factor(torch.from_numpy(H).cuda(), lam_rel=0.01)
    assert e.value.status == 3


# -------------------------------------------------------------------- sweep --
@pytest.mark.parametrize("out,n,bits,group,block", [
    (256, 512, 4, 0, 128),
    (203, 520, 4, 0, 128),
    (77, 640, 4, 128, 128),
    (130, 512, 3, 128, 64),
    (64, 384, 2, 64, 64),
    (33, 256, 3, 32, 128),
    (40, 512, 4, 256, 128),
    (57, 512, 3, 128, 32),
    (50, 200, 8, 0, 16),
    (70, 256, 2, 16, 32),
    # several super-blocks (1024 columns at B = 128, 512 below): the next
    # super-block's update, the far update beside the sweeps, the two-buffer
    # errors, a ragged last super-block, and groups wider than a super-block
    (48, 2688, 4, 128, 128),
    (40, 2560, 3, 0, 128),
    (32, 4096, 4, 2048, 128),
    (36, 1600, 4, 64, 64),
])
def test_sweep_matches_oracle(ctx, out, n, bits, group, block):
    print("sweep", out, n, bits, group, block, flush=True)
    H = _spd(n, 11 + n)
    Hl, lam = o.damp(H, lam_rel=0.01)
    U32 = o.factor_u(Hl).astype(np.float32)
    U = U32.astype(np.float64)
    g = torch.Generator().manual_seed(out * 7 + n)
    W = (torch.randn((out, n), generator=g) * 0.02).to(torch.float32)
    res = ctx.quantize(W.cuda(), torch.from_numpy(U32).cuda(), bits, group, block, lam, want_err=True)
    Wn = W.numpy().astype(np.float64)
    info = check_sweep(res, Wn, U, bits, group, block, H, lam)
    # E from the GPU equals the oracle's (same codes after replay) to fp32 accuracy
    rep = o.gptq_sweep(Wn, U, bits, group, block, replay=dict(codes=np32(res["codes"]), zeros=np32(res["zeros"]).astype(np.float32)))
    Eg = np32(res["err"]).astype(np.float64)
    assert np.abs(Eg - rep["E"]).max() <= 1e-3 * np.abs(rep["E"]).max()
    assert res["J_lam"] == pytest.approx(np.sum(rep["E"] ** 2), rel=1e-4)
    print(info)


def test_identity_hessian_is_round_to_nearest(ctx):
    n, out = 256, 100
    U32 = (np.eye(n) / np.sqrt(2.0)).astype(np.float32)
    g = torch.Generator().manual_seed(3)
    W = (torch.randn((out, n), generator=g) * 0.02).to(torch.float32)
    res = ctx.quantize(W.cuda(), torch.from_numpy(U32).cuda(), 4, 64, 64, 1.0)
    Wn = W.numpy().astype(np.float64)
    for k in range(n // 64):
        s = np32(res["scales"])[:, k].astype(np.float64)
        z = np32(res["zeros"])[:, k].astype(np.float64)
        grid = s[:, None, None] * (np.arange(16)[None, None, :] - z[:, None, None])
        best = np.abs(Wn[:, 64 * k:64 * k + 64, None] - grid).argmin(-1)
        assert np.array_equal(np32(res["codes"])[:, 64 * k:64 * k + 64], best)


def test_sweep_rejects_bad_arguments(ctx):
    W = torch.zeros((8, 64), device="cuda")
    U = torch.eye(64, device="cuda")
    for bits, group, block, status in [(1, 0, 64, 1), (9, 0, 64, 1), (4, 24, 64, 1), (4, 0, 48, 4), (4, 12, 64, 4)]:
        with pytest.raises(GPTQError) as e:
            ctx.quantize(W, U, bits, group, block, 0.1)
        assert e.value.status == status, (bits, group, block)


# --------------------------------------------------------------- end to end --
@pytest.mark.parametrize("name", ["single", "single_ragged", "square", "mlp"])
def test_layer_end_to_end(ctx, name):
    for spec in synth.SMALL[name]:
        print("layer", name, spec.name, flush=True)
        lay = synth.layer(spec)
        X = lay["X"].cuda()
        W = lay["W"].cuda()
        H = ctx.hessian(X)
        U, info, lam = ctx.factor(H, lam_rel=spec.lam_rel)
        res = ctx.quantize(W, U, spec.bits, spec.group, spec.block, lam)
        Hr = o.hessian(_bits(lay["X"]))
        Hl, lam_r = o.damp(Hr, lam_rel=spec.lam_rel)
        Ur = o.factor_u(Hl)
        assert np.linalg.norm(np32(H) - Hr) / np.linalg.norm(Hr) <= 1e-5
        assert lam == pytest.approx(lam_r, rel=1e-5)
        rep = {}
        check_sweep(res, lay["W"].numpy().astype(np.float64), Ur, spec.bits, spec.group, spec.block, Hr, lam_r,
                    report=rep)
        print(spec.name, rep)


def test_layer_repeatable_bitwise(ctx):
    spec = synth.SMALL["square"][0]
    lay = synth.layer(spec, "cuda")
    outs = []
    for _ in range(2):
        H = ctx.hessian(lay["X"])
        U, _, lam = ctx.factor(H, lam_rel=spec.lam_rel)
        r = ctx.quantize(lay["W"], U, spec.bits, spec.group, spec.block, lam, want_err=True)
        outs.append([H.clone(), U.clone(), r["codes"].clone(), r["scales"].clone(), r["zeros"].clone(),
                     r["err"].clone(), r["J"], r["J_lam"]])
    a, b = outs
    for x, y in zip(a[:6], b[:6]):
        assert torch.equal(x, y)
    assert a[6] == b[6] and a[7] == b[7]


# ------------------------------------------------------------------- LoRA ---
LORA_SPECS = [synth.SMALL["lora"][0],
              # two 64-blocks in the Gram factorization (the second partial),
              # ragged last row block (400 = 6 * 64 + 16)
              synth.LayerSpec("lora96", 160, 400, 8192, 3, 0, 128, 1e-4, kind="lowrank", rank=96, seed=5),
              # rank at the limit, two full 64-blocks
              synth.LayerSpec("lora128", 96, 640, 8192, 3, 0, 128, 1e-4, kind="lowrank", rank=128, seed=6),
              # power-law spectra (eigenvalue ratio lambda_r / lambda_{r+1} of a few percent or
              # less): the top-r subspace is still unique, but a plain r-column iteration
              # would need thousands of steps to find it
              synth.LayerSpec("pow16", 160, 384, 8192, 3, 0, 128, 1e-4, decay=0.5, rank=16, seed=7),
              synth.LayerSpec("pow48", 120, 256, 6000, 4, 64, 64, 1e-4, decay=0.5, rank=48, seed=8),
              # damping a hundred times below the pages' smallest (the augmented Hessian
              # is singular without it): the Cholesky route against the oracle's eig + QR
              synth.LayerSpec("lam1e-6", 160, 384, 8192, 3, 0, 128, 1e-6, kind="lowrank", rank=16, seed=4),
              synth.LayerSpec("pow16-lam1e-6", 160, 384, 8192, 3, 0, 128, 1e-6, decay=0.5, rank=16, seed=7)]


@pytest.mark.parametrize("spec", LORA_SPECS, ids=lambda s: s.name)
def test_lora_matches_oracle(ctx, spec):
    print("lora", spec.name, spec.n, spec.rank, flush=True)
    lay = synth.layer(spec)
    res = ctx.lora(lay["W"].cuda(), lay["X"].cuda(), spec.rank, spec.bits, spec.group, spec.block,
                   lam_rel=spec.lam_rel)
    Hr = o.hessian(_bits(lay["X"]))
    Wn = lay["W"].numpy().astype(np.float64)
    ref = o.lora(Wn, Hr, spec.rank, spec.bits, spec.group, spec.block, lam_rel=spec.lam_rel)
    codes = np32(res["codes"])
    zeros = np32(res["zeros"]).astype(np.float32)
    agree = float(np.mean(codes == ref["codes"]))
    rep = o.lora(Wn, Hr, spec.rank, spec.bits, spec.group, spec.block, lam_rel=spec.lam_rel,
                 replay=dict(codes=codes, zeros=zeros))
    L = np32(res["L"]).astype(np.float64)
    R = np32(res["R"]).astype(np.float64)
    # L spans the top-r eigenspace: same projector as the oracle's
    P_g = L @ L.T
    P_r = ref["L"] @ ref["L"].T
    ev = np.sort(np.linalg.eigvalsh(Hr))[::-1]
    print(dict(agree=agree, forced=rep["forced_codes"], J=res["J"], J_ref=ref["J"], converged=res["converged"],
               gap=float(ev[spec.rank - 1] / ev[spec.rank]), proj=float(np.abs(P_g - P_r).max())))
    assert res["converged"]
    assert np.abs(L.T @ L - np.eye(spec.rank)).max() < 1e-5
    assert np.abs(P_g - P_r).max() < 1e-5
    assert agree >= 0.995
    assert np.array_equal(rep["codes"], codes)
    LR_g = R.T @ L.T  # [out, n] = R_out V^T
    LR_r = rep["R_out"] @ rep["L"].T
    assert np.linalg.norm(LR_g - LR_r) <= 1e-3 * np.linalg.norm(LR_r)
    assert abs(res["J"] - ref["J"]) <= 5e-3 * ref["J"]
    # the intrinsic correction lowers the objective against plain GPTQ (expected)
    Hl, _ = o.damp(Hr, lam_rel=spec.lam_rel)
    g = o.gptq_sweep(Wn, o.factor_u(Hl), spec.bits, spec.group, spec.block)
    assert res["J"] < o.objective(Wn, g["What"], Hr)


def test_lora_reports_an_iteration_that_stopped_at_its_cap(ctx):
    # r = 128 on a power-law spectrum: the subspace cannot be wider than r, so it
    # converges at lambda_129 / lambda_128 per step and stops at its cap; every
    # output is still written from the last Ritz vectors
    spec = synth.LayerSpec("pow128", 96, 384, 4096, 3, 0, 128, 1e-4, decay=0.5, rank=128, seed=9)
    lay = synth.layer(spec)
    res = ctx.lora(lay["W"].cuda(), lay["X"].cuda(), spec.rank, spec.bits, spec.group, spec.block,
                   lam_rel=spec.lam_rel)
    assert not res["converged"]
    L = np32(res["L"]).astype(np.float64)
    assert np.all(np.isfinite(L)) and np.all(np.isfinite(np32(res["R"])))
    assert np.abs(L.T @ L - np.eye(spec.rank)).max() < 1e-5
    Hr = o.hessian(_bits(lay["X"]))
    ev = np.sort(np.linalg.eigvalsh(Hr))[::-1]
    # a near-top subspace: its Rayleigh quotient sum is within 1e-3 of the optimum
    ritz = float(np.trace(L.T @ Hr @ L))
    print(dict(J=res["J"], ritz=ritz, opt=float(ev[:spec.rank].sum())), flush=True)
    assert ritz >= (1 - 1e-3) * ev[:spec.rank].sum()
    Wn = lay["W"].numpy().astype(np.float64)
    Hl, _ = o.damp(Hr, lam_rel=spec.lam_rel)
    g = o.gptq_sweep(Wn, o.factor_u(Hl), spec.bits, spec.group, spec.block)
    assert res["J"] < o.objective(Wn, g["What"], Hr)


# ---------------------------------------------------------------- batched ---
def test_batched_equals_single_calls(ctx):
    specs = synth.SMALL["vit"] + synth.SMALL["mlp"]
    lays = [synth.layer(s, "cuda") for s in specs]
    layers = [dict(W=l["W"], X=l["X"], bits=s.bits, group=s.group, block=s.block, lam_rel=s.lam_rel)
              for s, l in zip(specs, lays)]
    ctx.quantize_batched(layers)
    for s, l, b in zip(specs, lays, layers):
        print("batched", s.name, flush=True)
        H = ctx.hessian(l["X"])
        U, _, lam = ctx.factor(H, lam_rel=s.lam_rel)
        r = ctx.quantize(l["W"], U, s.bits, s.group, s.block, lam)
        assert torch.equal(H, b["H"]), s.name
        assert torch.equal(U, b["U"]), s.name
        assert torch.equal(r["codes"], b["codes"]), s.name
        assert torch.equal(r["zeros"], b["zeros"]), s.name
        assert torch.equal(r["scales"], b["scales"]), s.name
        assert r["J"] == b["J"] and r["J_lam"] == b["J_lam"]


def test_batched_matches_oracle(ctx):
    specs = synth.SMALL["vit"][:4]
    lays = [synth.layer(s) for s in specs]
    layers = [dict(W=l["W"].cuda(), X=l["X"].cuda(), bits=s.bits, group=s.group, block=s.block,
                   lam_rel=s.lam_rel) for s, l in zip(specs, lays)]
    ctx.quantize_batched(layers)
    for s, l, b in zip(specs, lays, layers):
        Hr = o.hessian(_bits(l["X"]))
        Hl, lam = o.damp(Hr, lam_rel=s.lam_rel)
        check_sweep(b, l["W"].numpy().astype(np.float64), o.factor_u(Hl), s.bits, s.group, s.block, Hr, lam)


def test_batched_factor_ragged_more_groups_than_cus(ctx):
    """40 layers of n = 450 (blocks of 64, the last one 2 wide, so the
    products take the general path): each pair step's panel launch has
    40 x 8 = 320 workgroups, more than the CUs, so the diagonal chains run
    once per problem first, the last pair's second block partial.  U must
    match the oracle and the single-layer factor bit for bit."""
    n, out, tokens = 450, 16, 1200
    layers = []
    for i in range(40):
        X = _rand_x(tokens, n, 700 + i)
        W = torch.from_numpy(np.random.default_rng(800 + i).normal(0.0, 0.02, size=(out, n)).astype(np.float32))
        layers.append(dict(W=W.cuda(), X=X.cuda(), bits=4, group=0, block=32, lam_rel=0.01))
    ctx.quantize_batched(layers)
    torch.cuda.synchronize()
    for i, b in enumerate(layers):
        assert b["info"] == 0, i
        Hn = np32(b["H"]).astype(np.float64)
        Hl, lam = o.damp(Hn, lam_rel=0.01)
        Ur = o.factor_u(Hl)
        Ug = np32(b["U"]).astype(np.float64)
        assert np.abs(Ug - Ur).max() <= 2e-6 * np.abs(Ur).max(), i
    for i in (0, 17, 39):
        U1, info, _ = ctx.factor(layers[i]["H"], lam_rel=0.01)
        assert info == 0 and torch.equal(U1, layers[i]["U"]), i


def test_batched_factor_more_groups_than_cus(ctx):
    """24 layers of n = 768 in one batched call: each step's panel launch has
    24 x 12 = 288 workgroups (one per CU), more than the chip's CUs, so the
    plan runs each pair's diagonal chain once per problem first and the panel
    groups load it.  Every U must match the oracle's factor of its own H, and
    the same bits as the single-layer factor (12 groups, each repeating the
    chain itself)."""
    n, out, tokens = 768, 32, 1536
    layers = []
    for i in range(24):
        X = _rand_x(tokens, n, 500 + i)
        W = torch.from_numpy(np.random.default_rng(600 + i).normal(0.0, 0.02, size=(out, n)).astype(np.float32))
        layers.append(dict(W=W.cuda(), X=X.cuda(), bits=4, group=64, block=64, lam_rel=0.01))
    ctx.quantize_batched(layers)
    torch.cuda.synchronize()
    for i, b in enumerate(layers):
        assert b["info"] == 0, i
        Hn = np32(b["H"]).astype(np.float64)
        Hl, lam = o.damp(Hn, lam_rel=0.01)
        Ur = o.factor_u(Hl)
        Ug = np32(b["U"]).astype(np.float64)
        assert np.abs(Ug - Ur).max() <= 2e-6 * np.abs(Ur).max(), i
    for i in (0, 11, 23):
        U1, info, _ = ctx.factor(layers[i]["H"], lam_rel=0.01)
        assert info == 0 and torch.equal(U1, layers[i]["U"]), i

"""GPU deployable outputs against the oracle, through the C ABI.

Packing and unpacking are integer work: bit-exact.  The low-rank factors'
codes, scales and zero points come from the same fp32 steps on both sides:
bit-exact too.  The W4A16 product is compared with the oracle's float64
product on bf16-rounded weights (the operands the matrix unit is given); the
products x w are exact in fp32 and the GPU sums K of them in fp32, so in any
order the error is at most gamma_K sum_k |x_k w_k| with gamma_K = K u / (1 - K u),
u = 2^-24.  Against the oracle's product on the unrounded weights a further
2^-8 sum |x w| (half a bf16 spacing per weight) is allowed.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gptq_ref as o  # noqa: E402
from post_weight_quantization_gptq_amd import Context, GPTQError, synth  # noqa: E402
from parity import np32  # noqa: E402

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def ctx():
    c = Context("cuda:0")
    yield c
    c.close()


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_pack_unpack_bit_exact(ctx, bits):
    r = np.random.default_rng(100 + bits)
    for rows, n in ((1, 1), (3, 7), (5, 61), (17, 130), (64, 4096)):
        q = r.integers(0, 1 << bits, (rows, n)).astype(np.uint8)
        print("pack", bits, rows, n, flush=True)
        P = ctx.pack_codes(torch.from_numpy(q).cuda(), bits)
        ref = o.pack_codes(q, bits)
        assert np.array_equal(np32(P).view(np.uint32), ref)
        back = ctx.unpack_codes(torch.from_numpy(ref.view(np.int32)).cuda(), n, bits)
        assert np.array_equal(np32(back), q)


def test_pack_ignores_bits_above_the_width(ctx):
    q = np.random.default_rng(7).integers(0, 256, (4, 50)).astype(np.uint8)
    P = ctx.pack_codes(torch.from_numpy(q).cuda(), 3)
    assert np.array_equal(np32(P).view(np.uint32), o.pack_codes(q & 7, 3))


def _lowrank_case(n, r, out, seed):
    g = np.random.default_rng(seed)
    L = g.normal(0, 0.1, (n, r)).astype(np.float32)
    R = g.normal(0, 0.02, (r, out)).astype(np.float32)
    L[:, 0] = np.abs(L[:, 0])  # an all-positive component (lo = 0)
    if r > 1:
        R[1] = -np.abs(R[1])  # an all-negative one (hi = 0)
    if r > 2:
        L[:, 2] = 0.0  # a degenerate one (s = 1, z = 0)
    return L, R


@pytest.mark.parametrize("n,r,out,bits,bits_R", [(64, 4, 48, 4, 4), (300, 16, 257, 8, 8), (2048, 64, 2048, 4, 8),
                                                 (1, 1, 1, 8, 8), (513, 3, 9, 2, 2), (96, 5, 200, 8, 3)])
def test_lowrank_quantisation_bit_exact(ctx, n, r, out, bits, bits_R):
    print("lowrank", n, r, out, bits, bits_R, flush=True)
    L, R = _lowrank_case(n, r, out, n + r + out)
    res = ctx.quantize_lowrank(torch.from_numpy(L).cuda(), torch.from_numpy(R).cuda(), bits, bits_R)
    ref = o.quantize_lowrank(L, R, bits, bits_R)
    for side in ("L", "R"):
        assert np.array_equal(np32(res[side + "_codes"]), ref[side + "_codes"]), side
        assert np.array_equal(np32(res[side + "_scales"]), ref[side + "_scales"].astype(np.float32)), side
        assert np.array_equal(np32(res[side + "_zeros"]), ref[side + "_zeros"].astype(np.uint8)), side
        assert np.array_equal(np32(res[side + "_hat"]).astype(np.float64), ref[side + "_hat"]), side


def test_lowrank_of_a_lora_run(ctx):
    # the factors the intrinsic LoRA returns, at 4 and 8 bits; the low-rank
    # product's error shrinks with the width
    spec = synth.LayerSpec("lr_deploy", 96, 256, 2048, 4, 0, 128, 0.01, kind="lowrank", rank=16, seed=90)
    lay = synth.layer(spec)
    res = ctx.lora(lay["W"].cuda(), lay["X"].cuda(), 16, spec.bits, spec.group, spec.block, lam_rel=spec.lam_rel)
    L, R = np32(res["L"]), np32(res["R"])
    errs = []
    for bits in (4, 8):
        q = ctx.quantize_lowrank(res["L"], res["R"], bits)
        ref = o.quantize_lowrank(L, R, bits)
        if bits == 4:  # and the pages' pairing, L at 4 bits with R at 8
            qm = ctx.quantize_lowrank(res["L"], res["R"], 4, 8)
            rm = o.quantize_lowrank(L, R, 4, 8)
            assert np.array_equal(np32(qm["R_codes"]), rm["R_codes"]) and np.array_equal(np32(qm["L_codes"]), rm["L_codes"])
        assert np.array_equal(np32(q["L_codes"]), ref["L_codes"]) and np.array_equal(np32(q["R_codes"]), ref["R_codes"])
        LR = L.astype(np.float64) @ R
        errs.append(np.abs(np32(q["L_hat"]).astype(np.float64) @ np32(q["R_hat"]) - LR).max() / np.abs(LR).max())
    print(dict(rel_err_4bit=errs[0], rel_err_8bit=errs[1]), flush=True)
    assert errs[1] < errs[0] < 0.5


def _gemm_case(M, N, K, group, seed):
    X = synth.w4a16_inputs(M, K, seed)
    codes, scales, zeros = synth.w4_stored(N, K, group, seed)
    return X, codes.numpy(), scales.numpy(), zeros.numpy()


def _check_gemm(Y, Xb, codes, scales, zeros, group, rows=None):
    """Y (numpy fp32 [len(rows), N]) against the oracle on the given rows of X."""
    Xf = o._as_f64(Xb) if rows is None else o._as_f64(Xb[rows])
    K = codes.shape[1]
    zf = zeros.astype(np.float32)
    ref_b = o.gemm_w4a16(Xf, codes, scales, zf, group, weight_bf16=True)
    ref = o.gemm_w4a16(Xf, codes, scales, zf, group)
    Wb = o.bf16_round(o.dequantize(codes, scales, zf, group).astype(np.float32)).astype(np.float64)
    mag = np.abs(Xf) @ np.abs(Wb).T
    gam = K * U32 / (1 - K * U32)
    e_b = np.abs(Y.astype(np.float64) - ref_b)
    e = np.abs(Y.astype(np.float64) - ref)
    info = dict(max_err_bf16w=float((e_b / mag).max()), gamma_K=gam, max_err=float((e / mag).max()),
                rel_fro=float(np.linalg.norm(Y - ref) / np.linalg.norm(ref)))
    print(info, flush=True)
    assert np.all(e_b <= gam * mag + 1e-30), info
    assert np.all(e <= (gam + 2.0 ** -8) * mag * 1.0001 + 1e-30), info
    return info


@pytest.mark.parametrize("M,N,K,group", [(1, 1, 32, 0), (100, 70, 96, 32), (300, 200, 256, 128), (257, 129, 512, 0),
                                         (513, 384, 1024, 64), (256, 128, 64, 16), (70, 260, 128, 128), (600, 130, 64, 8),
                                         (1100, 256, 256, 0), (64, 40, 96, 96),
                                         # up to 128 rows: the split-K few-row kernel
                                         (2, 300, 512, 128), (5, 129, 256, 8), (16, 100, 64, 0), (3, 17, 32, 32),
                                         (16, 1024, 4096, 128), (17, 64, 128, 64), (8, 64, 256, 0), (4, 48, 416, 32),
                                         (40, 200, 512, 128), (128, 96, 256, 16), (129, 64, 128, 0)])
def test_gemm_w4a16_matches_oracle(ctx, M, N, K, group):
    print("gemm", M, N, K, group, flush=True)
    X, codes, scales, zeros = _gemm_case(M, N, K, group, M + N + K)
    P = torch.from_numpy(o.pack_codes(codes, 4).view(np.int32)).cuda()
    Y = ctx.gemm_w4a16(X.cuda(), P, torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(), group)
    _check_gemm(np32(Y), synth.bits_to_numpy(X), codes, scales, zeros, group)


def test_gemm_w4a16_pitched_output_and_input(ctx):
    import ctypes
    M, N, K, group = 130, 96, 128, 32
    X, codes, scales, zeros = _gemm_case(M, N, K, group, 5)
    Xw = torch.zeros((M, K + 40), dtype=torch.int16)
    Xw[:, :K] = X
    Xd = Xw.cuda()
    P = torch.from_numpy(o.pack_codes(codes, 4).view(np.int32)).cuda()
    S, Z = torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda()
    Yw = torch.full((M, N + 7), 7.0, device="cuda")
    vp = ctypes.c_void_p
    ctx._check(ctx.lib.gptq_gemm_w4a16(ctx.handle, vp(Xd.data_ptr()), M, K + 40, vp(P.data_ptr()), vp(S.data_ptr()),
                                       vp(Z.data_ptr()), N, K, group, vp(Yw.data_ptr()), N + 7))
    assert ctx.lib.gptq_gemm_w4a16(ctx.handle, None, 0, 0, None, None, None, 0, 0, 0, None, 0) == 0  # M == 0
    torch.cuda.synchronize()
    Yn = np32(Yw)
    assert np.all(Yn[:, N:] == 7.0)  # outside the M x N part untouched
    _check_gemm(Yn[:, :N], synth.bits_to_numpy(X), codes, scales, zeros, group)
    # the binding with a pitched view of X
    Y2 = ctx.gemm_w4a16(Xd[:, :K], P, S, Z, group)
    assert torch.equal(Y2, Yw[:, :N])


def test_gemm_w4a16_of_a_gptq_layer(ctx):
    # end to end on the GPU: the sweep's codes, packed by the library, then the
    # product; against the oracle on the same codes
    spec = synth.LayerSpec("w4_e2e", 192, 512, 4096, 4, 128, 128, 0.01, decay=0.4, outlier_channels=4, seed=91)
    lay = synth.layer(spec)
    X = lay["X"].cuda()
    H = ctx.hessian(X)
    U, _, lam = ctx.factor(H, lam_rel=spec.lam_rel)
    q = ctx.quantize(lay["W"].cuda(), U, 4, 128, 128, lam)
    P = ctx.pack_codes(q["codes"], 4)
    Y = ctx.gemm_w4a16(X[:1000], P, q["scales"], q["zeros"], 128)
    codes, scales, zeros = np32(q["codes"]), np32(q["scales"]), np32(q["zeros"])
    _check_gemm(np32(Y), synth.bits_to_numpy(lay["X"][:1000]), codes, scales, zeros, 128)


@pytest.mark.parametrize("bits", [2, 3, 8])
@pytest.mark.parametrize("M,N,K,group", [(1, 1, 32, 0), (100, 70, 96, 32), (300, 200, 256, 128), (513, 384, 1024, 64),
                                         (600, 130, 64, 8), (129, 64, 128, 0), (200, 129, 160, 16),
                                         # up to 128 rows: the split-K few-row kernel, K % 128 tails included
                                         (5, 129, 256, 8), (16, 100, 64, 0), (17, 64, 128, 64), (4, 48, 416, 32),
                                         (128, 96, 352, 16), (16, 1024, 4096, 128)])
def test_gemm_wqa16_matches_oracle(ctx, M, N, K, group, bits):
    # codes of 2, 3 and 8 bits: every 8-code chunk position of a 32-code step
    # (the 3-bit chunks straddle words), groups from 8 codes to the whole row
    print("gemm_wq", M, N, K, group, bits, flush=True)
    X = synth.w4a16_inputs(M, K, M + N + K + bits)
    codes, scales, zeros = (t.numpy() for t in synth.wq_stored(N, K, group, bits, M + N + K))
    P = torch.from_numpy(o.pack_codes(codes, bits).view(np.int32)).cuda()
    assert P.shape[1] == K * bits // 32
    Y = ctx.gemm_wqa16(X.cuda(), P, torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(), group, bits)
    _check_gemm(np32(Y), synth.bits_to_numpy(X), codes, scales, zeros, group)


@pytest.mark.parametrize("M", [16, 600])
def test_gemm_wqa16_at_4_bits_is_the_w4a16_product(ctx, M):
    # the general entry at 4 bits runs the W4A16 kernels: the same bits
    X, codes, scales, zeros = _gemm_case(M, 200, 512, 128, 11)
    P = torch.from_numpy(o.pack_codes(codes, 4).view(np.int32)).cuda()
    S, Z, Xd = torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(), X.cuda()
    assert torch.equal(ctx.gemm_wqa16(Xd, P, S, Z, 128, 4), ctx.gemm_w4a16(Xd, P, S, Z, 128))


@pytest.mark.parametrize("bits,group", [(3, 128), (2, 64)])
def test_gemm_wqa16_of_a_gptq_layer(ctx, bits, group):
    # the widths of the MLP (3-bit g128) and ViT (2-bit g64) layers, end to
    # end on the GPU: the sweep's codes packed by the library, then the product
    spec = synth.LayerSpec("wq_e2e", 160, 512, 4096, bits, group, 128, 0.01, decay=1.0, outlier_channels=0,
                           seed=92 + bits)
    lay = synth.layer(spec)
    X = lay["X"].cuda()
    H = ctx.hessian(X)
    U, _, lam = ctx.factor(H, lam_rel=spec.lam_rel)
    q = ctx.quantize(lay["W"].cuda(), U, bits, group, 128, lam)
    P = ctx.pack_codes(q["codes"], bits)
    for M in (40, 1000):  # the few-row and the tiled kernel
        Y = ctx.gemm_wqa16(X[:M], P, q["scales"], q["zeros"], group, bits)
        codes, scales, zeros = np32(q["codes"]), np32(q["scales"]), np32(q["zeros"])
        _check_gemm(np32(Y), synth.bits_to_numpy(lay["X"][:M]), codes, scales, zeros, group)


@pytest.mark.parametrize("bits", [2, 3, 8])
def test_gemm_wqa16_pitched_repeatable_and_empty(ctx, bits):
    # pitched X and Y, repeated calls bitwise equal, and K = 0 writing zeros,
    # at each width the general entry adds
    M, N, K, group = 300, 130, 256, 64
    X, _, _, _ = _gemm_case(M, N, K, group, 5 + bits)
    codes, scales, zeros = (t.numpy() for t in synth.wq_stored(N, K, group, bits, 5))
    P = torch.from_numpy(o.pack_codes(codes, bits).view(np.int32)).cuda()
    S, Z = torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda()
    Xw = torch.zeros((M, K + 24), dtype=torch.int16, device="cuda")
    Xw[:, :K] = X.cuda()
    Yw = torch.full((M, N + 7), 5.0, device="cuda")
    for rows in (M, 40):  # the tiled and the few-row kernel
        ctx.gemm_wqa16(Xw[:rows], P, S, Z, group, bits, K=K, Y=Yw[:rows])
        assert torch.all(Yw[:rows, N:] == 5.0)  # nothing written past N
        _check_gemm(np32(Yw[:rows, :N]), synth.bits_to_numpy(X[:rows]), codes, scales, zeros, group)
        Y1 = Yw[:rows, :N].clone()
        for _ in range(2):
            assert torch.equal(ctx.gemm_wqa16(Xw[:rows, :K], P, S, Z, group, bits), Y1)
    Y0 = torch.full((5, 3), 9.0, device="cuda")
    ctx.gemm_wqa16(torch.zeros((5, 8), dtype=torch.int16, device="cuda"), torch.zeros((3, 0), dtype=torch.int32,
                   device="cuda"), torch.ones((3, 1), device="cuda"), torch.zeros((3, 1), dtype=torch.uint8,
                   device="cuda"), 0, bits, K=0, Y=Y0)
    assert torch.count_nonzero(Y0).item() == 0


def test_gemm_wqa16_rejects_other_widths(ctx):
    X = torch.zeros((8, 64), dtype=torch.int16, device="cuda")
    S = torch.ones((4, 1), device="cuda")
    Z = torch.zeros((4, 1), dtype=torch.uint8, device="cuda")
    for bits in (1, 5, 6, 7, 9):
        P = torch.zeros((4, 64 * bits // 32), dtype=torch.int32, device="cuda")
        with pytest.raises(GPTQError):
            ctx.gemm_wqa16(X, P, S, Z, 0, bits)


@pytest.mark.parametrize("M", [16, 100, 600])
def test_gemm_w4a16_is_bitwise_repeatable(ctx, M):
    # fixed summation orders in both kernels (no atomics): repeated calls
    # give the same bits
    X, codes, scales, zeros = _gemm_case(M, 256, 512, 64, 3)
    P = torch.from_numpy(o.pack_codes(codes, 4).view(np.int32)).cuda()
    S, Z, Xd = torch.from_numpy(scales).cuda(), torch.from_numpy(zeros).cuda(), X.cuda()
    Y1 = ctx.gemm_w4a16(Xd, P, S, Z, 64)
    for _ in range(3):
        assert torch.equal(ctx.gemm_w4a16(Xd, P, S, Z, 64), Y1)


def test_gemm_w4a16_empty_sum_is_zero(ctx):
    X = torch.zeros((5, 8), dtype=torch.int16, device="cuda")
    P = torch.zeros((3, 0), dtype=torch.int32, device="cuda")
    Y = torch.full((5, 3), 9.0, device="cuda")
    ctx.gemm_w4a16(X, P, torch.ones((3, 1), device="cuda"), torch.zeros((3, 1), dtype=torch.uint8, device="cuda"), 0,
                   K=0, Y=Y)
    assert torch.count_nonzero(Y).item() == 0


def test_gemm_w4a16_rejects_unsupported(ctx):
    X = torch.zeros((8, 48), dtype=torch.int16, device="cuda")
    P = torch.zeros((4, 6), dtype=torch.int32, device="cuda")
    S = torch.ones((4, 1), device="cuda")
    Z = torch.zeros((4, 1), dtype=torch.uint8, device="cuda")
    with pytest.raises(GPTQError):
        ctx.gemm_w4a16(X, P, S, Z, 0)  # K % 32 != 0
    X = torch.zeros((8, 96), dtype=torch.int16, device="cuda")
    P = torch.zeros((4, 12), dtype=torch.int32, device="cuda")
    with pytest.raises(GPTQError):
        ctx.gemm_w4a16(X, P, torch.ones((4, 2), device="cuda"), torch.zeros((4, 2), dtype=torch.uint8, device="cuda"),
                       48)  # group not a power of two
    # code rows not 16-byte aligned (a view one word into its buffer)
    Pw = torch.zeros((4 * 12 + 1,), dtype=torch.int32, device="cuda")[1:].view(4, 12)
    with pytest.raises(GPTQError):
        ctx.gemm_w4a16(X, Pw, torch.ones((4, 1), device="cuda"), torch.zeros((4, 1), dtype=torch.uint8, device="cuda"), 0)

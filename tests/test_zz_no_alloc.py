"""The no-allocation quantise entry point against gptq_quantize.

gptq_quantize_noalloc runs the same kernels as gptq_quantize with every
intermediate in the library's fixed per-device scratch array, so its outputs
must equal gptq_quantize's bit for bit.  Calls run back to back, each
following one with a smaller layer, so that anything the array keeps from
the call before (working weights, block errors, per-row sums) would show.
"""
import pytest

torch = pytest.importorskip("torch")

from post_weight_quantization_gptq_amd import Context, GPTQError  # noqa: E402

pytestmark = pytest.mark.gpu

# (out, n, bits, group, block): the largest layers the array holds first,
# then ragged smaller ones
CASES = [
    (1024, 1024, 4, 128, 128),
    (256, 4096, 3, 64, 16),
    (200, 384, 3, 0, 32),
    (77, 136, 8, 8, 64),
]


def _layer(out, n, seed):
    g = torch.Generator().manual_seed(seed)
    X = (torch.randn((max(2 * n, 256), n), generator=g)).to(torch.bfloat16).view(torch.int16)
    W = torch.randn((out, n), generator=g) * 0.05
    return W, X


def _outputs(out, n, group):
    ng = n // group if group else 1
    return dict(codes=torch.full((out, n), 0xEE, dtype=torch.uint8, device="cuda:0"),
                scales=torch.full((out, ng), float("nan"), dtype=torch.float32, device="cuda:0"),
                zeros=torch.full((out, ng), 0xEE, dtype=torch.uint8, device="cuda:0"),
                err=torch.full((out, n), float("nan"), dtype=torch.float32, device="cuda:0"))


def test_noalloc_equals_quantize_back_to_back():
    ctx = Context("cuda:0")
    try:
        for i, (out, n, bits, group, block) in enumerate(CASES):
            print("noalloc case", out, n, bits, group, block, flush=True)
            W, X = _layer(out, n, 100 + i)
            H = ctx.hessian(X.cuda())
            U, info, lam = ctx.factor(H, lam_rel=0.01)
            assert info == 0
            Wd = W.cuda()
            ref = ctx.quantize(Wd, U, bits, group, block, lam, want_err=True)
            got = ctx.quantize_noalloc(Wd, U, bits, group, block, lam, _outputs(out, n, group), want_err=True)
            torch.cuda.synchronize()
            for k in ("codes", "scales", "zeros", "err"):
                assert torch.equal(got[k], ref[k]), k
            assert got["J"] == ref["J"] and got["J_lam"] == ref["J_lam"]
            assert int(got["codes"].max()) <= (1 << bits) - 1
    finally:
        ctx.close()


def test_noalloc_rejects_layers_past_its_limits():
    ctx = Context("cuda:0")
    try:
        for out, n in ((1025, 64), (64, 4104), (512, 4096)):
            W = torch.zeros((out, n), dtype=torch.float32, device="cuda:0")
            U = torch.eye(n, dtype=torch.float32, device="cuda:0")
            with pytest.raises(GPTQError) as e:
                ctx.quantize_noalloc(W, U, 4, 8, 16, 0.0, _outputs(out, n, 8))
            assert "no-allocation limits" in str(e.value)
        # a small layer still works on the same context afterwards
        out, n = 33, 64
        W, X = _layer(out, n, 7)
        U, info, lam = ctx.factor(ctx.hessian(X.cuda()), lam_rel=0.01)
        Wd = W.cuda()
        ref = ctx.quantize(Wd, U, 4, 16, 16, lam)
        got = ctx.quantize_noalloc(Wd, U, 4, 16, 16, lam, _outputs(out, n, 16))
        torch.cuda.synchronize()
        for k in ("codes", "scales", "zeros"):
            assert torch.equal(got[k], ref[k]), k
    finally:
        ctx.close()

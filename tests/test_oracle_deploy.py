"""Pins of the oracle's deployable outputs: packed codes against independent
layouts (nibbles at 4 bits, bytes at 8 bits, a hand-worked 3-bit row) and the
round trip; low-precision L and R against per-vector round-to-nearest; the
dequant GEMM against the dequantised weights' product.  CPU only.
"""
import numpy as np
import pytest

from oracle import gptq_ref as o


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_pack_round_trip(bits):
    r = np.random.default_rng(bits)
    for n in (1, 7, 32, 61, 130):
        q = r.integers(0, 1 << bits, (3, n)).astype(np.uint8)
        p = o.pack_codes(q, bits)
        assert p.shape == (3, (n * bits + 31) // 32)
        assert np.array_equal(o.unpack_codes(p, n, bits), q)


def test_pack_4bit_is_nibbles_and_8bit_is_bytes():
    r = np.random.default_rng(9)
    q4 = r.integers(0, 16, (2, 40)).astype(np.uint8)
    p4 = o.pack_codes(q4, 4)
    for k in range(40):
        assert np.array_equal((p4[:, k // 8] >> (4 * (k % 8))) & 0xF, q4[:, k])
    q8 = r.integers(0, 256, (2, 12)).astype(np.uint8)
    assert np.array_equal(o.pack_codes(q8, 8).view(np.uint8).reshape(2, 12), q8)  # little-endian bytes


def test_pack_3bit_hand_worked_row():
    # codes 1..7, 0, 1, 2, 3 at 3 bits: bit offsets 0, 3, ..., 30; the last
    # code (3 = 0b011) straddles the word boundary (bits 30, 31 | 32)
    q = np.array([[1, 2, 3, 4, 5, 6, 7, 0, 1, 2, 3]], dtype=np.uint8)
    w0 = (1 | 2 << 3 | 3 << 6 | 4 << 9 | 5 << 12 | 6 << 15 | 7 << 18 | 0 << 21 | 1 << 24 | 2 << 27
          | (3 & 0b11) << 30)
    assert o.pack_codes(q, 3).tolist() == [[w0, 0]]
    q[0, 10] = 4  # 0b100: only bit 32 set
    assert o.pack_codes(q, 3).tolist() == [[w0 & 0x3FFFFFFF, 1]]


def test_lowrank_quantisation_is_per_vector_rounding():
    r = np.random.default_rng(10)
    L = r.normal(0, 0.1, (40, 6))
    R = r.normal(0, 0.02, (6, 30))
    for bits in (4, 8):
        res = o.quantize_lowrank(L, R, bits)
        maxq = (1 << bits) - 1
        for k in range(6):
            for vec, codes, s, z in ((L[:, k], res["L_codes"][:, k], res["L_scales"][k], res["L_zeros"][k]),
                                     (R[k], res["R_codes"][k], res["R_scales"][k], res["R_zeros"][k])):
                # the grid spans [min(v, 0), max(v, 0)] and every value goes to
                # its nearest level (fp32)
                lo, hi = min(vec.min(), 0), max(vec.max(), 0)
                assert np.float32(s) == np.float32((np.float32(hi) - np.float32(lo)) / np.float32(maxq))
                levels = (np.float32(s) * (np.arange(maxq + 1, dtype=np.float32) - np.float32(z))).astype(np.float64)
                best = np.abs(vec[:, None] - levels[None, :]).argmin(axis=1)
                near = np.abs(np.abs(vec[:, None] - levels[None, :]).min(axis=1) - s / 2) < 1e-6 * s
                assert np.all((codes == best) | near)
        err8 = np.abs(res["L_hat"] - L).max() if bits == 8 else None
    assert err8 is not None and err8 <= 0.5 * (L.max() - min(L.min(), 0)) / 255 * 1.001


def test_dequant_gemm_is_the_product_of_the_dequantised_weights():
    r = np.random.default_rng(11)
    X = r.normal(0, 1, (9, 64)).astype(np.float32).astype(np.float64)
    q = r.integers(0, 16, (5, 64)).astype(np.uint8)
    s = r.uniform(0.01, 0.1, (5, 2)).astype(np.float32)
    z = r.integers(0, 16, (5, 2)).astype(np.float32)
    Y = o.gemm_w4a16(X, q, s, z, group=32)
    Wd = np.zeros((5, 64))
    for i in range(5):
        for k in range(64):
            g = k // 32
            Wd[i, k] = float(np.float32(s[i, g]) * np.float32(float(q[i, k]) - z[i, g]))
    assert np.abs(Y - X @ Wd.T).max() <= 1e-12 * np.abs(Y).max()


def test_bf16_round_matches_torch_and_hand_worked_ties():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(12)
    v = np.concatenate([r.normal(0, 1, 4000), r.normal(0, 1e-30, 500), r.normal(0, 1e30, 500),
                        [0.0, -0.0, 1.0, -2.5, 3.0e38]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(o.bf16_round(v).view(np.uint32), ref.view(np.uint32))
    # the spacing of bf16 at 1 is 2^-7: 1 + 2^-8 is a tie going to the even 1;
    # 1 + 3 2^-8 a tie going to the even 1 + 2^-6; just above a tie rounds up
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8)], dtype=np.float32)
    assert o.bf16_round(ties).tolist() == [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0]


def test_dequant_gemm_with_bf16_weights():
    # weights of the form s (q - z) with s a power of two are exact in bf16,
    # so both forms agree exactly; otherwise each weight moves by at most half
    # a bf16 spacing (2^-8 relative)
    r = np.random.default_rng(13)
    X = r.normal(0, 1, (7, 64))
    q = r.integers(0, 16, (6, 64)).astype(np.uint8)
    z = r.integers(0, 16, (6, 2)).astype(np.float32)
    s2 = (2.0 ** r.integers(-8, 0, (6, 2))).astype(np.float32)
    assert np.array_equal(o.gemm_w4a16(X, q, s2, z, 32, weight_bf16=True), o.gemm_w4a16(X, q, s2, z, 32))
    s = r.uniform(0.01, 0.1, (6, 2)).astype(np.float32)
    Wd = o.dequantize(q, s, z, 32)
    Wb = (o.gemm_w4a16(np.eye(64), q, s, z, 32, weight_bf16=True)).T
    assert np.all(np.abs(Wb - Wd) <= 2.0 ** -8 * np.abs(Wd))
    assert np.abs(Wb - Wd).max() > 0


def test_lowrank_mixed_widths_take_each_factor_at_its_own_width():
    # [LoRA] results: L and R at 4 and 8 bits respectively
    r = np.random.default_rng(14)
    L, R = r.normal(0, 0.1, (30, 5)), r.normal(0, 0.02, (5, 20))
    mixed, a, b = o.quantize_lowrank(L, R, 4, 8), o.quantize_lowrank(L, R, 4), o.quantize_lowrank(L, R, 8)
    for k in ("codes", "scales", "zeros", "hat"):
        assert np.array_equal(mixed["L_" + k], a["L_" + k]) and np.array_equal(mixed["R_" + k], b["R_" + k])
    assert mixed["L_codes"].max() <= 15 and mixed["R_codes"].max() > 15

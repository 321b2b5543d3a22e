"""The C-ABI library loads and exports every entry point its header declares.

CPU only: nothing here launches a kernel.  Calls that fail validation before any
HIP call (a null context) are exercised too.
"""
import ctypes
import os

import pytest

import post_weight_quantization_gptq_amd as g


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g.library_path()):
        from post_weight_quantization_gptq_amd import build_lib
        build_lib.build()
    return g.load_library()


def test_header_declares_the_pass():
    names = g.exported_symbols()
    for need in ("gptq_create", "gptq_destroy", "gptq_strerror", "gptq_last_error", "gptq_hessian",
                 "gptq_factor", "gptq_quantize", "gptq_lora", "gptq_quantize_batched", "gptq_hessian64",
                 "gptq_olrc", "gptq_bid_up", "gptq_lora_refine", "gptq_round_2d", "gptq_quantize_qronos",
                 "gptq_cross_gram", "gptq_pack_codes", "gptq_unpack_codes", "gptq_quantize_lowrank",
                 "gptq_gemm_w4a16"):
        assert need in names


def test_library_exports_every_declared_symbol(lib):
    for name in g.exported_symbols():
        assert hasattr(lib, name), name


def test_library_exports_nothing_else(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", g.library_path()], capture_output=True, text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    gptq = {s for s in syms if s.startswith("gptq_")}
    assert gptq == set(g.exported_symbols())


def test_null_context_is_rejected_without_a_gpu(lib):
    assert lib.gptq_hessian(None, None, 0, 0, 0, None, 0) == 1
    assert lib.gptq_quantize(None, None, 0, 0, None, 4, 0, 128, 0.0, None, None, None, None, None) == 1
    info = ctypes.c_int32(0)
    assert lib.gptq_factor(None, None, 0, 0.0, 0.0, None, ctypes.byref(info), None) == 1
    assert lib.gptq_gemm_w4a16(None, None, 0, 0, None, None, None, 0, 0, 0, None, 0) == 1
    assert lib.gptq_pack_codes(None, None, 0, 0, 4, None) == 1
    assert lib.gptq_destroy(None) == 1
    assert lib.gptq_create(None, 0, None) == 1
    assert lib.gptq_strerror(2) == b"damped Hessian is not positive definite"
    assert lib.gptq_last_error(None) == b""


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        g.load_library(str(tmp_path / "missing.so"))

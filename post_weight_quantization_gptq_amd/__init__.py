"""MI355X-native GPTQ layer quantization.

A thin Python binding (ctypes) over ``libgptq_mi355x.so``, the HIP/C library
declared in ``include/gptq.h``.  This module only marshals arguments: it checks
shapes and dtypes, allocates output tensors with torch (device memory) and
passes raw pointers and the current HIP stream to the library, where every step
of the pass runs.  There is no fallback: if the library is missing, every entry
point raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GPTQError",
    "Context",
    "library_path",
    "load_library",
    "exported_symbols",
    "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBNAME = "libgptq_mi355x.so"
_lib = None

STATUS = {
    0: "GPTQ_OK",
    1: "GPTQ_ERR_INVALID_ARG",
    2: "GPTQ_ERR_NOT_PD",
    3: "GPTQ_ERR_NONFINITE",
    4: "GPTQ_ERR_UNSUPPORTED",
    5: "GPTQ_ERR_HIP",
    6: "GPTQ_ERR_NO_MEMORY",
    7: "GPTQ_ERR_NOT_CONVERGED",
}
NOT_CONVERGED = 7


class GPTQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), msg))
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, _LIBNAME)


class _Layer(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p),
        ("tokens", ctypes.c_int64),
        ("ldx", ctypes.c_int64),
        ("W", ctypes.c_void_p),
        ("out", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("pad0", ctypes.c_int32),
        ("lam_abs", ctypes.c_double),
        ("lam_rel", ctypes.c_double),
        ("H", ctypes.c_void_p),
        ("U", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("zeros", ctypes.c_void_p),
        ("err", ctypes.c_void_p),
        ("obj", ctypes.c_double * 2),
        ("info", ctypes.c_int32),
        ("pad1", ctypes.c_int32),
    ]


def load_library(path: str | None = None):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(
            "%s is not built; run `python -m post_weight_quantization_gptq_amd.build_lib`" % p)
    L = ctypes.CDLL(p)
    vp, i32, i64, d = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    L.gptq_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp]
    L.gptq_destroy.argtypes = [vp]
    L.gptq_strerror.argtypes = [ctypes.c_int]
    L.gptq_strerror.restype = ctypes.c_char_p
    L.gptq_last_error.argtypes = [vp]
    L.gptq_last_error.restype = ctypes.c_char_p
    L.gptq_hessian.argtypes = [vp, vp, i64, i32, i64, vp, ctypes.c_int]
    L.gptq_factor.argtypes = [vp, vp, i32, d, d, vp, ctypes.POINTER(i32), ctypes.POINTER(d)]
    L.gptq_quantize.argtypes = [vp, vp, i32, i32, vp, i32, i32, i32, d, vp, vp, vp, vp,
                                ctypes.POINTER(d)]
    L.gptq_quantize_noalloc.argtypes = L.gptq_quantize.argtypes
    L.gptq_lora.argtypes = [vp, vp, i32, i32, vp, i64, i64, i32, i32, i32, i32, d, d,
                            vp, vp, vp, vp, vp, ctypes.POINTER(d), ctypes.POINTER(i32)]
    L.gptq_lora_refine.argtypes = [vp, vp, i32, i32, vp, i64, i64, i32, i32, i32, i32, d, d, i32,
                                   vp, vp, vp, vp, vp, ctypes.POINTER(d), ctypes.POINTER(i32)]
    L.gptq_hessian64.argtypes = [vp, vp, i64, i32, i64, vp]
    L.gptq_olrc.argtypes = [vp, vp, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp, vp, ctypes.POINTER(d)]
    L.gptq_bid_up.argtypes = [vp, vp, i32, i32, vp, i32, vp, vp, i32, i32, i32, vp, vp, vp,
                              ctypes.POINTER(d)]
    L.gptq_round_2d.argtypes = [vp, vp, i32, i32, vp, vp, i32, i32, vp, vp, ctypes.POINTER(d)]
    L.gptq_cross_gram.argtypes = [vp, vp, vp, i64, i32, i64, vp]
    L.gptq_quantize_qronos.argtypes = [vp, vp, i32, i32, vp, vp, i64, i64, i32, i32, i32, d, d, vp, vp, vp, vp,
                                       ctypes.POINTER(d), ctypes.POINTER(i32)]
    L.gptq_pack_codes.argtypes = [vp, vp, i32, i32, i32, vp]
    L.gptq_unpack_codes.argtypes = [vp, vp, i32, i32, i32, vp]
    L.gptq_quantize_lowrank.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.gptq_gemm_w4a16.argtypes = [vp, vp, i64, i64, vp, vp, vp, i32, i32, i32, vp, i64]
    L.gptq_gemm_wqa16.argtypes = [vp, vp, i64, i64, vp, vp, vp, i32, i32, i32, i32, vp, i64]
    L.gptq_quantize_batched.argtypes = [vp, i32, ctypes.POINTER(_Layer)]
    L.gptq_timing.argtypes = [vp, ctypes.c_char_p]
    L.gptq_kernel_time.argtypes = [vp, ctypes.c_char_p, ctypes.POINTER(d), ctypes.POINTER(i64)]
    for name in ("gptq_create", "gptq_destroy", "gptq_hessian", "gptq_factor", "gptq_quantize",
                 "gptq_quantize_noalloc", "gptq_lora", "gptq_lora_refine", "gptq_hessian64", "gptq_olrc", "gptq_bid_up", "gptq_round_2d",
                 "gptq_quantize_qronos", "gptq_cross_gram", "gptq_pack_codes", "gptq_unpack_codes",
                 "gptq_quantize_lowrank", "gptq_gemm_w4a16", "gptq_gemm_wqa16",
                 "gptq_quantize_batched", "gptq_timing", "gptq_kernel_time"):
        getattr(L, name).restype = ctypes.c_int
    if path is None:
        _lib = L
    return L


def exported_symbols(header: str | None = None):
    """Function names declared in include/gptq.h."""
    import re
    header = header or os.path.join(os.path.dirname(_HERE), "include", "gptq.h")
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gptq_[a-z0-9_]+)\s*\(", txt)))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


class Context:
    """A library context bound to a device and to the current torch stream."""

    def __init__(self, device=None):
        import torch
        self.torch = torch
        self.lib = load_library()
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        if dev.type != "cuda":
            raise ValueError("the GPTQ library needs a GPU device")
        self.device = torch.device("cuda", dev.index if dev.index is not None else torch.cuda.current_device())
        self.stream = torch.cuda.current_stream(self.device)
        h = ctypes.c_void_p()
        self._check(self.lib.gptq_create(ctypes.byref(h), self.device.index, ctypes.c_void_p(self.stream.cuda_stream)),
                    ctx=None)
        self.handle = h

    def timing(self, kernels: str | None = "*"):
        """Start per-kernel event timing of `kernels` (comma-separated names or
        "*"), clearing the totals; None stops it."""
        self._check(self.lib.gptq_timing(self.handle, None if kernels is None else kernels.encode()))

    def kernel_time(self, name: str):
        """(total ms, launches) of the kernel `name` since timing was enabled."""
        ms, cnt = ctypes.c_double(0.0), ctypes.c_int64(0)
        self._check(self.lib.gptq_kernel_time(self.handle, name.encode(), ctypes.byref(ms), ctypes.byref(cnt)))
        return ms.value, cnt.value

    def close(self):
        if getattr(self, "handle", None):
            self.lib.gptq_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    # ------------------------------------------------------------------ util
    def _check(self, rc, ctx="self"):
        if rc != 0:
            msg = ""
            if ctx is not None and getattr(self, "handle", None):
                msg = (self.lib.gptq_last_error(self.handle) or b"").decode()
            if not msg:
                msg = self.lib.gptq_strerror(rc).decode()
            raise GPTQError(rc, msg)

    def _check_conv(self, rc) -> bool:
        """_check, except that a subspace iteration stopped at its cap (every
        output written) gives False instead of raising."""
        if rc == NOT_CONVERGED:
            return False
        self._check(rc)
        return True

    def _dev(self, t, dtype, name):
        torch = self.torch
        if t.device != self.device:
            raise ValueError("%s must be on %s" % (name, self.device))
        if t.dtype != dtype:
            raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        return t

    def _xbits(self, X):
        torch = self.torch
        if X.dtype == torch.bfloat16:
            X = X.view(torch.int16)
        if X.dtype not in (torch.int16, torch.uint16):
            raise TypeError("X must be bfloat16 (or its int16 bit patterns)")
        if X.dim() != 2 or X.stride(1) != 1:
            raise ValueError("X must be a row-major [tokens, ldx] matrix")
        if X.device != self.device:
            raise ValueError("X must be on %s" % self.device)
        return X

    # ----------------------------------------------------------- entry points
    def hessian(self, X, n: int | None = None, H=None, accumulate: bool = False):
        """H = (accumulate ? H : 0) + X^T X (fp32 [n, n])."""
        torch = self.torch
        X = self._xbits(X)
        tokens, ldx = X.shape[0], X.stride(0)
        n = X.shape[1] if n is None else int(n)
        if H is None:
            H = torch.empty((n, n), dtype=torch.float32, device=self.device)
        self._dev(H, torch.float32, "H")
        self._check(self.lib.gptq_hessian(self.handle, _ptr(X), tokens, n, ldx, _ptr(H), int(bool(accumulate))))
        return H

    def factor(self, H, lam_abs: float = 0.0, lam_rel: float = 0.01, U=None):
        """U upper with (H + lam I)^{-1} = U^T U.  Returns (U, info, lam); raises on failure."""
        torch = self.torch
        self._dev(H, torch.float32, "H")
        n = H.shape[0]
        if U is None:
            U = torch.empty((n, n), dtype=torch.float32, device=self.device)
        info = ctypes.c_int32(0)
        lam = ctypes.c_double(0.0)
        rc = self.lib.gptq_factor(self.handle, _ptr(H), n, float(lam_abs), float(lam_rel), _ptr(U),
                                  ctypes.byref(info), ctypes.byref(lam))
        if rc == 2:
            err = GPTQError(rc, (self.lib.gptq_last_error(self.handle) or b"").decode())
            err.info = info.value
            raise err
        self._check(rc)
        return U, info.value, lam.value

    def quantize(self, W, U, bits: int, group: int, block: int, lam: float, want_err: bool = False,
                 out=None):
        """Blocked GPTQ sweep.  Returns dict(codes, scales, zeros, err, J, J_lam)."""
        torch = self.torch
        self._dev(W, torch.float32, "W")
        self._dev(U, torch.float32, "U")
        o, n = W.shape
        ng = n // group if group else 1
        if out is None:
            out = dict(codes=torch.empty((o, n), dtype=torch.uint8, device=self.device),
                       scales=torch.empty((o, ng), dtype=torch.float32, device=self.device),
                       zeros=torch.empty((o, ng), dtype=torch.uint8, device=self.device),
                       err=torch.empty((o, n), dtype=torch.float32, device=self.device) if want_err else None)
        obj = (ctypes.c_double * 2)()
        self._check(self.lib.gptq_quantize(self.handle, _ptr(W), o, n, _ptr(U), int(bits), int(group), int(block),
                                           float(lam), _ptr(out["codes"]), _ptr(out["scales"]), _ptr(out["zeros"]),
                                           _ptr(out.get("err")), obj))
        res = dict(out)
        res["J"], res["J_lam"] = obj[0], obj[1]
        return res

    def quantize_noalloc(self, W, U, bits: int, group: int, block: int, lam: float, out, want_err: bool = False):
        """quantize() through the entry point that allocates nothing: the outputs are
        caller-provided tensors in ``out`` (codes, scales, zeros and optionally err)."""
        torch = self.torch
        self._dev(W, torch.float32, "W")
        self._dev(U, torch.float32, "U")
        o, n = W.shape
        obj = (ctypes.c_double * 2)()
        self._check(self.lib.gptq_quantize_noalloc(self.handle, _ptr(W), o, n, _ptr(U), int(bits), int(group),
                                                   int(block), float(lam), _ptr(out["codes"]), _ptr(out["scales"]),
                                                   _ptr(out["zeros"]), _ptr(out.get("err") if want_err else None),
                                                   obj))
        res = dict(out)
        res["J"], res["J_lam"] = obj[0], obj[1]
        return res

    def lora(self, W, X, r: int, bits: int, group: int, block: int, lam_abs: float = 0.0,
             lam_rel: float = 1e-4):
        """GPTQ-intrinsic LoRA.  Returns dict(codes, scales, zeros, L [n, r], R [r, out], J, J_lam, info,
        converged); converged is False when the top-r subspace iteration stopped at its cap."""
        torch = self.torch
        self._dev(W, torch.float32, "W")
        X = self._xbits(X)
        o, n = W.shape
        ng = n // group if group else 1
        res = dict(codes=torch.empty((o, n), dtype=torch.uint8, device=self.device),
                   scales=torch.empty((o, ng), dtype=torch.float32, device=self.device),
                   zeros=torch.empty((o, ng), dtype=torch.uint8, device=self.device),
                   L=torch.empty((n, r), dtype=torch.float32, device=self.device),
                   R=torch.empty((r, o), dtype=torch.float32, device=self.device))
        obj = (ctypes.c_double * 2)()
        info = ctypes.c_int32(0)
        conv = self._check_conv(self.lib.gptq_lora(self.handle, _ptr(W), o, n, _ptr(X), X.shape[0], X.stride(0),
                                                   int(r), int(bits), int(group), int(block), float(lam_abs),
                                                   float(lam_rel), _ptr(res["codes"]), _ptr(res["scales"]),
                                                   _ptr(res["zeros"]), _ptr(res["L"]), _ptr(res["R"]), obj,
                                                   ctypes.byref(info)))
        res["J"], res["J_lam"], res["info"], res["converged"] = obj[0], obj[1], info.value, conv
        return res

    def lora_refine(self, W, X, r: int, bits: int, group: int, block: int, rounds: int = 1,
                    lam_abs: float = 0.0, lam_rel: float = 1e-4):
        """Intrinsic LoRA, then `rounds` of OLrC + Bid-Up and a last OLrC.
        Returns dict(codes, scales, zeros, L [n, r], R [r, out], trace [2 rounds + 2])."""
        torch = self.torch
        self._dev(W, torch.float32, "W")
        X = self._xbits(X)
        o, n = W.shape
        ng = n // group if group else 1
        res = dict(codes=torch.empty((o, n), dtype=torch.uint8, device=self.device),
                   scales=torch.empty((o, ng), dtype=torch.float32, device=self.device),
                   zeros=torch.empty((o, ng), dtype=torch.uint8, device=self.device),
                   L=torch.empty((n, r), dtype=torch.float32, device=self.device),
                   R=torch.empty((r, o), dtype=torch.float32, device=self.device))
        tr = (ctypes.c_double * (2 * int(rounds) + 2))()
        info = ctypes.c_int32(0)
        conv = self._check_conv(self.lib.gptq_lora_refine(
            self.handle, _ptr(W), o, n, _ptr(X), X.shape[0], X.stride(0), int(r), int(bits), int(group), int(block),
            float(lam_abs), float(lam_rel), int(rounds), _ptr(res["codes"]), _ptr(res["scales"]), _ptr(res["zeros"]),
            _ptr(res["L"]), _ptr(res["R"]), tr, ctypes.byref(info)))
        res["trace"], res["info"], res["converged"] = list(tr), info.value, conv
        return res

    def hessian64(self, X, n: int | None = None, H=None):
        """H = X^T X accurate to fp64 rounding (fp64 [n, n])."""
        torch = self.torch
        X = self._xbits(X)
        n = X.shape[1] if n is None else int(n)
        if H is None:
            H = torch.empty((n, n), dtype=torch.float64, device=self.device)
        self._dev(H, torch.float64, "H")
        self._check(self.lib.gptq_hessian64(self.handle, _ptr(X), X.shape[0], n, X.stride(0), _ptr(H)))
        return H

    def olrc(self, W, H, r: int, bits: int, group: int, codes, scales, zeros):
        """Optimal rank-r compensation for fixed codes.  Returns dict(L [n, r], R [r, out], J, converged)."""
        torch = self.torch
        self._dev(W, torch.float32, "W")
        self._dev(H, torch.float64, "H")
        self._dev(codes, torch.uint8, "codes")
        self._dev(scales, torch.float32, "scales")
        self._dev(zeros, torch.uint8, "zeros")
        o, n = W.shape
        res = dict(L=torch.empty((n, r), dtype=torch.float32, device=self.device),
                   R=torch.empty((r, o), dtype=torch.float32, device=self.device))
        J = ctypes.c_double(0.0)
        conv = self._check_conv(self.lib.gptq_olrc(self.handle, _ptr(W), o, n, _ptr(H), int(r), int(bits),
                                                   int(group), _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(res["L"]),
                                                   _ptr(res["R"]), ctypes.byref(J)))
        res["J"], res["converged"] = J.value, conv
        return res

    def bid_up(self, W, H, L, R, bits: int, group: int, block: int, codes, scales, zeros):
        """One Bid-Up pass; rewrites codes in place.  Returns the objective after the pass."""
        torch = self.torch
        self._dev(W, torch.float32, "W")
        self._dev(H, torch.float64, "H")
        self._dev(L, torch.float32, "L")
        self._dev(R, torch.float32, "R")
        self._dev(codes, torch.uint8, "codes")
        self._dev(scales, torch.float32, "scales")
        self._dev(zeros, torch.uint8, "zeros")
        o, n = W.shape
        J = ctypes.c_double(0.0)
        self._check(self.lib.gptq_bid_up(self.handle, _ptr(W), o, n, _ptr(H), int(L.shape[1]), _ptr(L), _ptr(R),
                                         int(bits), int(group), int(block), _ptr(codes), _ptr(scales), _ptr(zeros),
                                         ctypes.byref(J)))
        return J.value

    def cross_gram(self, X, Y, G=None):
        """G = X^T Y (fp32 [n, n])."""
        torch = self.torch
        X = self._xbits(X)
        Y = self._xbits(Y)
        if Y.shape != X.shape or Y.stride(0) != X.stride(0):
            raise ValueError("X and Y must have the same shape and row pitch")
        n = X.shape[1]
        if G is None:
            G = torch.empty((n, n), dtype=torch.float32, device=self.device)
        self._dev(G, torch.float32, "G")
        self._check(self.lib.gptq_cross_gram(self.handle, _ptr(X), _ptr(Y), X.shape[0], n, X.stride(0), _ptr(G)))
        return G

    def quantize_qronos(self, W, X, Xq, bits: int, group: int, block: int, lam_abs: float = 0.0,
                        lam_rel: float = 0.01, want_target: bool = False):
        """GPTQ with the quantised-input target.  Returns dict(codes, scales, zeros, Wt or None, J, J_lam, info)."""
        torch = self.torch
        self._dev(W, torch.float32, "W")
        X = self._xbits(X)
        Xq = self._xbits(Xq)
        if Xq.shape != X.shape or Xq.stride(0) != X.stride(0):
            raise ValueError("X and Xq must have the same shape and row pitch")
        o, n = W.shape
        ng = n // group if group else 1
        res = dict(codes=torch.empty((o, n), dtype=torch.uint8, device=self.device),
                   scales=torch.empty((o, ng), dtype=torch.float32, device=self.device),
                   zeros=torch.empty((o, ng), dtype=torch.uint8, device=self.device),
                   Wt=torch.empty((o, n), dtype=torch.float32, device=self.device) if want_target else None)
        obj = (ctypes.c_double * 2)()
        info = ctypes.c_int32(0)
        self._check(self.lib.gptq_quantize_qronos(self.handle, _ptr(W), o, n, _ptr(X), _ptr(Xq), X.shape[0],
                                                  X.stride(0), int(bits), int(group), int(block), float(lam_abs),
                                                  float(lam_rel), _ptr(res["codes"]), _ptr(res["scales"]),
                                                  _ptr(res["zeros"]), _ptr(res["Wt"]), obj, ctypes.byref(info)))
        res["J"], res["J_lam"], res["info"] = obj[0], obj[1], info.value
        return res

    def round_2d(self, X, UG, UH, qmin: int, qmax: int, want_delta: bool = False):
        """GPTQ-2D two-sided rounding of X [m, n] with the factors UG [m, m], UH [n, n].
        Returns dict(Z int32 [m, n], delta fp32 [m, n] or None, J)."""
        torch = self.torch
        self._dev(X, torch.float32, "X")
        self._dev(UG, torch.float32, "UG")
        self._dev(UH, torch.float32, "UH")
        m, n = X.shape
        Z = torch.empty((m, n), dtype=torch.int32, device=self.device)
        D = torch.empty((m, n), dtype=torch.float32, device=self.device) if want_delta else None
        J = ctypes.c_double(0.0)
        self._check(self.lib.gptq_round_2d(self.handle, _ptr(X), m, n, _ptr(UG), _ptr(UH), int(qmin), int(qmax),
                                           _ptr(Z), _ptr(D), ctypes.byref(J)))
        return dict(Z=Z, delta=D, J=J.value)

    def pack_codes(self, codes, bits: int):
        """codes uint8 [rows, n] -> int32 [rows, ceil(n bits / 32)] holding the
        uint32 code words (little-endian bitstream per row)."""
        torch = self.torch
        self._dev(codes, torch.uint8, "codes")
        rows, n = codes.shape
        P = torch.empty((rows, (n * bits + 31) // 32), dtype=torch.int32, device=self.device)
        self._check(self.lib.gptq_pack_codes(self.handle, _ptr(codes), rows, n, int(bits), _ptr(P)))
        return P

    def unpack_codes(self, packed, n: int, bits: int):
        torch = self.torch
        self._dev(packed, torch.int32, "packed")
        rows = packed.shape[0]
        if packed.shape[1] != (n * bits + 31) // 32:
            raise ValueError("packed has the wrong number of words per row")
        codes = torch.empty((rows, n), dtype=torch.uint8, device=self.device)
        self._check(self.lib.gptq_unpack_codes(self.handle, _ptr(packed), rows, int(n), int(bits), _ptr(codes)))
        return codes

    def quantize_lowrank(self, L, R, bits: int, bits_R: int | None = None, want_hat: bool = True):
        """Round-to-nearest of L [n, r] at `bits` and R [r, out] at `bits_R` (default: the
        same), one grid per rank component.
        Returns dict(L_codes, L_scales, L_zeros, L_hat, R_codes, R_scales, R_zeros, R_hat)."""
        torch = self.torch
        self._dev(L, torch.float32, "L")
        self._dev(R, torch.float32, "R")
        n, r = L.shape
        if R.shape[0] != r:
            raise ValueError("L and R have different ranks")
        out = R.shape[1]
        dev = self.device
        res = dict(L_codes=torch.empty((n, r), dtype=torch.uint8, device=dev),
                   L_scales=torch.empty(r, dtype=torch.float32, device=dev),
                   L_zeros=torch.empty(r, dtype=torch.uint8, device=dev),
                   L_hat=torch.empty((n, r), dtype=torch.float32, device=dev) if want_hat else None,
                   R_codes=torch.empty((r, out), dtype=torch.uint8, device=dev),
                   R_scales=torch.empty(r, dtype=torch.float32, device=dev),
                   R_zeros=torch.empty(r, dtype=torch.uint8, device=dev),
                   R_hat=torch.empty((r, out), dtype=torch.float32, device=dev) if want_hat else None)
        self._check(self.lib.gptq_quantize_lowrank(
            self.handle, _ptr(L), _ptr(R), n, r, out, int(bits), int(bits if bits_R is None else bits_R),
            _ptr(res["L_codes"]), _ptr(res["L_scales"]),
            _ptr(res["L_zeros"]), _ptr(res["L_hat"]), _ptr(res["R_codes"]), _ptr(res["R_scales"]),
            _ptr(res["R_zeros"]), _ptr(res["R_hat"])))
        return res

    def gemm_w4a16(self, X, packed, scales, zeros, group: int, K: int | None = None, Y=None):
        """Y = X What^T (fp32 [M, N]) from bf16 X [M, K] and 4-bit packed codes [N, K/8]."""
        torch = self.torch
        X = self._xbits(X)
        self._dev(packed, torch.int32, "packed")
        self._dev(scales, torch.float32, "scales")
        self._dev(zeros, torch.uint8, "zeros")
        M = X.shape[0]
        K = int(K if K is not None else X.shape[1])
        N = packed.shape[0]
        if packed.shape[1] != K // 8:
            raise ValueError("packed must hold K/8 words per row")
        if Y is None:
            Y = torch.empty((M, N), dtype=torch.float32, device=self.device)
        self._dev(Y, torch.float32, "Y")
        self._check(self.lib.gptq_gemm_w4a16(self.handle, _ptr(X), M, X.stride(0), _ptr(packed), _ptr(scales),
                                             _ptr(zeros), N, K, int(group), _ptr(Y), Y.stride(0)))
        return Y

    def gemm_wqa16(self, X, packed, scales, zeros, group: int, bits: int, K: int | None = None, Y=None):
        """Y = X What^T (fp32 [M, N]) from bf16 X [M, K] and codes of `bits` bits (2, 3, 4 or 8) packed
        [N, K bits/32]."""
        torch = self.torch
        X = self._xbits(X)
        self._dev(packed, torch.int32, "packed")
        self._dev(scales, torch.float32, "scales")
        self._dev(zeros, torch.uint8, "zeros")
        M = X.shape[0]
        K = int(K if K is not None else X.shape[1])
        N = packed.shape[0]
        if K % 32 == 0 and packed.shape[1] != K * int(bits) // 32:
            raise ValueError("packed must hold K*bits/32 words per row")
        if Y is None:
            Y = torch.empty((M, N), dtype=torch.float32, device=self.device)
        self._dev(Y, torch.float32, "Y")
        self._check(self.lib.gptq_gemm_wqa16(self.handle, _ptr(X), M, X.stride(0), _ptr(packed), _ptr(scales),
                                             _ptr(zeros), N, K, int(group), int(bits), _ptr(Y), Y.stride(0)))
        return Y

    def quantize_batched(self, layers):
        """layers: list of dicts with W, bits, group, block, lam_rel (and X or H, optional lam_abs,
        err or want_err).
        Fills H/U/codes/scales/zeros per layer (allocating what is missing); returns the list."""
        torch = self.torch
        arr = (_Layer * len(layers))()
        keep = []
        for i, ly in enumerate(layers):
            W = self._dev(ly["W"], torch.float32, "W")
            o, n = W.shape
            g = int(ly["group"])
            ng = n // g if g else 1
            ly.setdefault("H", torch.empty((n, n), dtype=torch.float32, device=self.device))
            ly.setdefault("U", torch.empty((n, n), dtype=torch.float32, device=self.device))
            ly.setdefault("codes", torch.empty((o, n), dtype=torch.uint8, device=self.device))
            ly.setdefault("scales", torch.empty((o, ng), dtype=torch.float32, device=self.device))
            ly.setdefault("zeros", torch.empty((o, ng), dtype=torch.uint8, device=self.device))
            if ly.get("want_err") and ly.get("err") is None:
                ly["err"] = torch.empty((o, n), dtype=torch.float32, device=self.device)
            X = ly.get("X")
            if X is not None:
                X = self._xbits(X)
            a = arr[i]
            a.X = X.data_ptr() if X is not None else None
            a.tokens = X.shape[0] if X is not None else 0
            a.ldx = X.stride(0) if X is not None else n
            a.W, a.out, a.n = W.data_ptr(), o, n
            a.bits, a.group, a.block = int(ly["bits"]), g, int(ly["block"])
            a.lam_abs, a.lam_rel = float(ly.get("lam_abs", 0.0)), float(ly.get("lam_rel", 0.01))
            a.H, a.U = ly["H"].data_ptr(), ly["U"].data_ptr()
            a.codes, a.scales, a.zeros = ly["codes"].data_ptr(), ly["scales"].data_ptr(), ly["zeros"].data_ptr()
            a.err = ly["err"].data_ptr() if ly.get("err") is not None else None
            keep.append(X)
        rc = self.lib.gptq_quantize_batched(self.handle, len(layers), arr)
        for i, ly in enumerate(layers):
            ly["J"], ly["J_lam"], ly["info"] = arr[i].obj[0], arr[i].obj[1], arr[i].info
        self._check(rc)
        return layers

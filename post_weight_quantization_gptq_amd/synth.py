"""Seeded synthetic layers shaped like the workloads the GPTQ pages quantise.

Input generation only: this module holds none of the method's arithmetic.  It
draws weights W (fp32, [out, n]) and calibration inputs X (bfloat16 bit
patterns, [tokens, n]) with the shapes, spectra and outliers of five layer
configurations, plus smaller versions of each for parity tests.  The same bytes
are fed to the oracle and to the GPU library.

Recipe (all seeded; Q is a Haar rotation: QR of an N(0,1) fp64 matrix with
columns sign-fixed by sign(diag R)):
  single    W [256, 512] N(0, 0.02^2), 0.5% of entries (655) x8;
            X [1024, 512] = (Z * i^-1/2) Q^T                      (4-bit, per row)
  square    W [4096, 4096] N(0, 0.02^2);
            X [262144, 4096] = (Z * i^-0.4) Q^T, 8 channels x sqrt(20) (4-bit, g128)
  mlp       gate/up W [6144, 2048], down W [2048, 6144];
            X_in [262144, 2048] = (Z * i^-1/2) Q^T (shared by gate and up),
            X_down = relu(Z' * i^-1/2 Q'^T)^2 with 6144 channels    (3-bit, g128)
  lora      W [2048, 2048]; X [65536, 2048] = A diag(sigma) V^T with A having
            orthonormal columns, V Haar, sigma_1..64 ~ N(1, 0.1),
            sigma_{64+i} = 0.05 i^-1/2                               (3-bit, r = 64)
  vit       12 x {qkv [2304, 768], proj [768, 768], fc1 [3072, 768],
            fc2 [768, 3072]}; one X per layer, [50176, 768] or [50176, 3072],
            (Z * i^-1/2) Q^T                                         (2-bit, g64)
  r2d       the square layer, plus Y [65536, 4096] = (Z * i^-1/2) Q^T for
            the second (output-side) Gram of the two-sided rounding
  qronos    the square layer, its X and Xq = bf16(X + N(0, (0.05 std X)^2))
            standing in for the inputs of an already-quantised network
  w4a16     the stored form of a 4-bit [4096, 4096] layer (codes uniform on
            0..15, per-(row, group of 128) scales U(0.005, 0.01) and zero
            points uniform on 0..15, the ranges a min-max grid gives on
            N(0, 0.02^2) weights) applied to 8192 tokens of the square layer's
            input recipe; the same stand-in at 2, 3 and 8 bits (codes and
            zero points uniform on 0..2^bits - 1) for the other widths
where Z has i.i.d. N(0, 1) entries and i = 1..n indexes the input channels.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass
class LayerSpec:
    name: str
    out: int
    n: int
    tokens: int
    bits: int
    group: int
    block: int
    lam_rel: float
    kind: str = "power"          # power | lowrank | relu2
    decay: float = 0.5           # std of channel i is i^-decay
    outlier_entries: float = 0.0  # fraction of W entries scaled x8
    outlier_channels: int = 0    # X channels scaled x sqrt(20)
    rank: int = 0                # intrinsic-LoRA rank
    seed: int = 0
    x_key: str = ""              # layers with the same key share X
    extra: dict = field(default_factory=dict)


def _specs_full():
    s = {}
    s["single"] = [LayerSpec("single", 256, 512, 1024, 4, 0, 128, 0.01, decay=0.5,
                             outlier_entries=0.005, seed=1)]
    s["square"] = [LayerSpec("square", 4096, 4096, 262144, 4, 128, 128, 0.01, decay=0.4,
                             outlier_channels=8, seed=2)]
    s["mlp"] = [LayerSpec("gate", 6144, 2048, 262144, 3, 128, 128, 0.01, decay=0.5, seed=31, x_key="mlp_in"),
                LayerSpec("up", 6144, 2048, 262144, 3, 128, 128, 0.01, decay=0.5, seed=32, x_key="mlp_in"),
                LayerSpec("down", 2048, 6144, 262144, 3, 128, 128, 0.01, kind="relu2", decay=0.5, seed=33)]
    s["lora"] = [LayerSpec("lora", 2048, 2048, 65536, 3, 0, 128, 1e-4, kind="lowrank", rank=64, seed=4)]
    # two-sided rounding: the square layer (its W as the target, its input
    # Gram on the right) and a second 4096-wide seeded matrix whose Gram
    # stands for the output-side factor on the left
    s["r2d"] = [s["square"][0],
                LayerSpec("r2d_out", 4096, 4096, 65536, 4, 0, 128, 0.01, decay=0.5, seed=5)]
    vit = []
    for blk in range(12):
        for j, (nm, o, n) in enumerate([("qkv", 2304, 768), ("proj", 768, 768), ("fc1", 3072, 768),
                                        ("fc2", 768, 3072)]):
            vit.append(LayerSpec("b%d.%s" % (blk, nm), o, n, 50176, 2, 64, 64, 0.01, decay=0.5,
                                 seed=500 + 4 * blk + j))
    s["vit"] = vit
    return s


def _specs_small():
    """Same structure at sizes the oracle finishes in seconds; ragged on purpose
    (rows not a multiple of 16/64, tokens not a multiple of 64, columns not a
    multiple of the block for the per-row case)."""
    s = {}
    s["single"] = [LayerSpec("single", 256, 512, 1024, 4, 0, 128, 0.01, decay=0.5,
                             outlier_entries=0.005, seed=1)]
    s["single_ragged"] = [LayerSpec("single_ragged", 203, 520, 3001, 4, 0, 128, 0.01, decay=0.5,
                                    outlier_entries=0.005, seed=11)]
    s["square"] = [LayerSpec("square", 203, 640, 6001, 4, 128, 128, 0.01, decay=0.4,
                             outlier_channels=8, seed=2)]
    s["mlp"] = [LayerSpec("gate", 150, 384, 4000, 3, 128, 128, 0.01, decay=0.5, seed=31, x_key="mlp_in"),
                LayerSpec("up", 150, 384, 4000, 3, 128, 128, 0.01, decay=0.5, seed=32, x_key="mlp_in"),
                LayerSpec("down", 96, 768, 4000, 3, 128, 128, 0.01, kind="relu2", decay=0.5, seed=33)]
    s["lora"] = [LayerSpec("lora", 160, 384, 8192, 3, 0, 128, 1e-4, kind="lowrank", rank=16, seed=4)]
    vit = []
    for blk in range(2):
        for j, (nm, o, n) in enumerate([("qkv", 384, 128), ("proj", 128, 128), ("fc1", 384, 128),
                                        ("fc2", 128, 384)]):
            vit.append(LayerSpec("b%d.%s" % (blk, nm), o, n, 2000, 2, 64, 64, 0.01, decay=0.5,
                                 seed=500 + 4 * blk + j))
    s["vit"] = vit
    return s


FULL = _specs_full()
SMALL = _specs_small()


def haar(n: int, seed: int) -> torch.Tensor:
    """Haar-distributed orthogonal n x n (fp64, CPU)."""
    g = torch.Generator().manual_seed(seed)
    A = torch.randn((n, n), generator=g, dtype=torch.float64)
    Q, R = torch.linalg.qr(A)
    return Q * torch.sign(torch.diagonal(R))[None, :]


def weights(spec: LayerSpec, device="cpu") -> torch.Tensor:
    g = torch.Generator().manual_seed(10_000 + spec.seed)
    W = torch.randn((spec.out, spec.n), generator=g, dtype=torch.float64) * 0.02
    if spec.outlier_entries:
        k = int(round(spec.outlier_entries * spec.out * spec.n))
        idx = torch.randperm(spec.out * spec.n, generator=g)[:k]
        W.view(-1)[idx] *= 8.0
    return W.to(torch.float32).to(device)


def _to_bits(x: torch.Tensor) -> torch.Tensor:
    """float32 -> bfloat16 (round to nearest even) -> int16 bit patterns."""
    return x.to(torch.bfloat16).view(torch.int16)


def calibration(spec: LayerSpec, device="cpu", chunk: int = 16384) -> torch.Tensor:
    """X [tokens, n] as bf16 bit patterns (int16), generated in chunks on `device`."""
    dev = torch.device(device)
    n, T = spec.n, spec.tokens
    # layers that share an input (x_key) share its seed; a stable digest of the key
    key_seed = spec.seed if not spec.x_key else sum((i + 1) * ord(ch) for i, ch in enumerate(spec.x_key)) + 7
    X = torch.empty((T, n), dtype=torch.int16, device=dev)
    gen = torch.Generator(device=dev).manual_seed(20_000 + key_seed)
    if spec.kind == "lowrank":
        r = spec.rank
        gs = torch.Generator().manual_seed(30_000 + key_seed)
        sig = torch.cat([1.0 + 0.1 * torch.randn(r, generator=gs, dtype=torch.float64),
                         0.05 * torch.arange(1, n - r + 1, dtype=torch.float64) ** -0.5])
        V = haar(n, 40_000 + key_seed)
        # A with orthonormal columns: QR of a Gaussian [T, n] (fp64 on the CPU)
        A = torch.randn((T, n), generator=gs, dtype=torch.float64)
        A, R = torch.linalg.qr(A)
        A = A * torch.sign(torch.diagonal(R))[None, :]
        M = (sig[:, None] * V.T)  # diag(sigma) V^T
        for t0 in range(0, T, chunk):
            blk = (A[t0:t0 + chunk] @ M).to(torch.float32).to(dev)
            X[t0:t0 + chunk] = _to_bits(blk)
        return X
    Q = haar(n, 40_000 + key_seed).to(torch.float32).to(dev)
    std = (torch.arange(1, n + 1, dtype=torch.float64) ** -spec.decay).to(torch.float32).to(dev)
    ch = None
    if spec.outlier_channels:
        gs = torch.Generator().manual_seed(50_000 + key_seed)
        ch = torch.randperm(n, generator=gs)[:spec.outlier_channels].to(dev)
    for t0 in range(0, T, chunk):
        m = min(chunk, T - t0)
        Z = torch.randn((m, n), generator=gen, device=dev, dtype=torch.float32)
        blk = (Z * std[None, :]) @ Q.T
        if spec.kind == "relu2":
            blk = torch.relu(blk) ** 2
        if ch is not None:
            blk[:, ch] *= math.sqrt(20.0)
        X[t0:t0 + m] = _to_bits(blk)
    return X


def perturbed(X: torch.Tensor, seed: int, scale: float = 0.05, chunk: int = 16384) -> torch.Tensor:
    """A seeded stand-in for the inputs an already-quantised network feeds the
    layer: X (bf16 bits) plus N(0, (scale * std(X))^2) noise, rounded back to
    bf16, chunk by chunk on X's device."""
    dev = X.device
    gen = torch.Generator(device=dev).manual_seed(60_000 + seed)
    out = torch.empty_like(X)
    s = None
    for t0 in range(0, X.shape[0], chunk):
        blk = X[t0:t0 + chunk].view(torch.bfloat16).to(torch.float32)
        if s is None:
            s = scale * float(blk.std())
        noise = torch.randn(blk.shape, generator=gen, device=dev, dtype=torch.float32) * s
        out[t0:t0 + chunk] = _to_bits(blk + noise)
    return out


def layer(spec: LayerSpec, device="cpu"):
    """dict(W fp32 [out, n], X int16 bf16-bits [tokens, n]) for one layer."""
    return dict(W=weights(spec, device), X=calibration(spec, device))


def bits_to_numpy(X: torch.Tensor) -> np.ndarray:
    """bf16 bit patterns (int16 tensor) -> uint16 numpy array (for the oracle)."""
    return X.detach().cpu().numpy().view(np.uint16)


def w4_stored(N: int, K: int, group: int, seed: int):
    """Seeded stand-in for a 4-bit layer's stored form: codes [N, K] uint8
    uniform on 0..15, scales [N, G] float32 U(0.005, 0.01), zeros [N, G] uint8
    uniform on 0..15 (G = K / group, 1 for group 0)."""
    g = torch.Generator().manual_seed(70_000 + seed)
    G = K // group if group else 1
    codes = torch.randint(0, 16, (N, K), generator=g, dtype=torch.int64).to(torch.uint8)
    scales = (0.005 + 0.005 * torch.rand((N, G), generator=g, dtype=torch.float64)).to(torch.float32)
    zeros = torch.randint(0, 16, (N, G), generator=g, dtype=torch.int64).to(torch.uint8)
    return codes, scales, zeros


def wq_stored(N: int, K: int, group: int, bits: int, seed: int):
    """The same stand-in for a layer stored at `bits` bits: codes and zero
    points uniform on 0..2^bits - 1, scales U(0.005, 0.01)."""
    g = torch.Generator().manual_seed(71_000 + 97 * bits + seed)
    G = K // group if group else 1
    top = 1 << bits
    codes = torch.randint(0, top, (N, K), generator=g, dtype=torch.int64).to(torch.uint8)
    scales = (0.005 + 0.005 * torch.rand((N, G), generator=g, dtype=torch.float64)).to(torch.float32)
    zeros = torch.randint(0, top, (N, G), generator=g, dtype=torch.int64).to(torch.uint8)
    return codes, scales, zeros


W4A16 = dict(M=8192, N=4096, K=4096, group=128)
W4A16_DECODE_M = 16  # the same layer applied to 16 tokens (a decode-sized batch)


def w4a16_inputs(M: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    """Activations X [M, K] (bf16 bits) from the square layer's input recipe."""
    spec = LayerSpec("w4a16_x", K, K, M, 4, 128, 128, 0.01, decay=0.4, outlier_channels=8 if K >= 64 else 0,
                     seed=seed)
    return calibration(spec, device)

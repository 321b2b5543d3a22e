"""Benchmark of the GPTQ layer-quantization pass on one MI355X.

One step = the whole pass for one layer on inputs already resident in HBM:
gptq_hessian (X^T X on bf16 MFMA) -> gptq_factor (damping, fp64 Cholesky and
triangular inverse) -> gptq_quantize (blocked column sweep, trailing updates,
objective).  The default workload is the square projection layer: W 4096x4096,
4-bit, group 128, block 128, 262144 calibration tokens.

Prints one JSON line (rank 0).  Extra objects: `roofline` for the dominant
kernel (the Hessian contraction, timed live with HIP events on the library's
stream), `cpu_baseline` (the float64 oracle timed on a bounded sample on the
host cores), per-stage times and algorithmic TFLOP/s.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # dense MFMA bf16, MI355X
PEAK_HBM_GBS = 8000.0
METRIC = "ms per layer + TFLOP/s (frac of MFMA peak), 4096×4096 4-bit g128 GPTQ"


def layer_flops(out, n, tokens, block, n_total=None):
    """Algorithmic flops of one layer (counted as in the design notes)."""
    nt = n_total or n
    syrk = tokens * n * (n + 1)
    factor = 2 * nt ** 3 / 3
    nblk = -(-n // block)
    sweep = 0
    trail = 0
    for b in range(nblk):
        b0, b1 = b * block, min((b + 1) * block, n)
        w = b1 - b0
        sweep += out * w * (w - 1)
        trail += 2 * out * w * (nt - b1)
    return dict(syrk=syrk, factor=factor, sweep=sweep, trail=trail, total=syrk + factor + sweep + trail)


def cpu_baseline(spec, lay, max_rows=512, tok_sample=32768):
    """The float64 oracle, as it stands, on a bounded sample of the same layer,
    scaled to ms per layer: Hessian on tok_sample tokens (scaled by tokens),
    the full damping + factor, and the sweep on max_rows rows (scaled by rows)."""
    import numpy as np
    from oracle import gptq_ref as o
    from post_weight_quantization_gptq_amd import synth
    Xs = synth.bits_to_numpy(lay["X"][:tok_sample].cpu())
    t0 = time.perf_counter()
    Hs = o.hessian(Xs)
    t_h = time.perf_counter() - t0
    # factor on a full-rank matrix of the same size (the sampled H is rank
    # deficient only through damping, which keeps it positive definite)
    t0 = time.perf_counter()
    Hl, lam = o.damp(Hs, lam_rel=spec.lam_rel)
    U = o.factor_u(Hl)
    t_f = time.perf_counter() - t0
    W = lay["W"][:max_rows].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    o.gptq_sweep(W, U, spec.bits, spec.group, spec.block)
    t_s = time.perf_counter() - t0
    total_ms = 1e3 * (t_h * spec.tokens / tok_sample + t_f + t_s * spec.out / max_rows)
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count()
    return {"value": round(total_ms, 1), "unit": "ms/layer", "cores": cores, "kind": "oracle",
            "blas": blas_vendor(),
            "sample": "Hessian on %d of %d tokens (x%.0f), full damping+factor (n=%d), sweep on %d of %d rows (x%.0f);"
                      " measured %.1f s + %.1f s + %.1f s" % (tok_sample, spec.tokens, spec.tokens / tok_sample,
                                                               spec.n, max_rows, spec.out, spec.out / max_rows,
                                                               t_h, t_f, t_s)}


def blas_vendor():
    """The BLAS numpy calls (name, version, and the library's own configuration line)."""
    import numpy as np
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return "%s %s (%s); threads %s" % (b.get("name"), b.get("version"), b.get("openblas configuration", "").strip(),
                                           os.environ.get("OMP_NUM_THREADS", os.environ.get("OPENBLAS_NUM_THREADS",
                                                                                            "default")))
    except Exception as e:  # pragma: no cover
        return "unknown (%s)" % e


def code_digest(path):
    """SHA-256 of a C/HIP source with its comments and whitespace removed, so
    that a counter record stays valid across edits of comments only."""
    import hashlib
    import re
    txt = open(path, encoding="utf-8").read()
    txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
    txt = re.sub(r"//[^\n]*", " ", txt)
    return hashlib.sha256(" ".join(txt.split()).encode()).hexdigest()


def kernel_traffic(kernel, workload, source):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_<workload>_traffic.json, or None when absent or taken on
    a different version of its source file's code."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (kernel, workload))
    src = os.path.join(ROOT, "post_weight_quantization_gptq_amd", "csrc", source)
    try:
        rec = json.load(open(path))
        if rec.get("source_code_sha256") != code_digest(src):
            return None
        return rec.get("bytes_per_launch")
    except Exception:
        return None


def syrk_traffic(workload):
    return kernel_traffic("k_syrk", workload, "syrk.hip")


def counter_rates(workload):
    """Counter-based rates of the layer's kernels from the committed rocprofv3
    records (profiles/*_<workload>_counters.json and the sweep's traffic
    record), each only while its source file's code is the one the counters
    were taken on.  Matrix-pipe shares are SQ_VALU_MFMA_BUSY_CYCLES over the
    cycles of the SIMDs (or, for the factor, of the CUs the kernel occupies);
    the clock is GRBM_GUI_ACTIVE per XCD over the kernel's duration."""
    out = {}

    def load(name, source):
        try:
            rec = json.load(open(os.path.join(ROOT, "profiles", name)))
            src = os.path.join(ROOT, "post_weight_quantization_gptq_amd", "csrc", source)
            return rec if rec.get("source_code_sha256") == code_digest(src) else None
        except Exception:
            return None

    def mean(xs):
        return round(sum(xs) / len(xs), 4) if xs else None

    rec = load("k_syrk_%s_counters.json" % workload, "syrk.hip")
    if rec:
        d = rec["dispatches"]
        out["k_syrk"] = {"mfma_busy": mean([x["mfma_busy"] for x in d]), "clock_GHz": mean([x["clock_GHz"] for x in d]),
                         "lds_active": mean([x["lds_active"] for x in d])}
    rec = load("k_trail_%s_counters.json" % workload, "sweep.hip")
    if rec:
        for ts in ("64", "128"):
            d = [x for x in rec["dispatches"] if x["kernel"].endswith("<%s>" % ts)]
            if d:
                out["k_trail<%s>" % ts] = {"mfma_busy": mean([x["mfma_busy"] for x in d]),
                                           "clock_GHz": mean([x["clock_GHz"] for x in d])}
    rec = load("k_sweep_%s_traffic.json" % workload, "sweep.hip")
    if rec:
        gbs = rec["hbm_GBps_under_profiler"]
        out["k_sweep"] = {"bytes_per_launch": rec["bytes_per_launch"], "gb_s": gbs, "peak": PEAK_HBM_GBS,
                          "frac": round(gbs / PEAK_HBM_GBS, 4)}
    rec = load("factor_%s_counters.json" % workload, "factor.hip")
    if rec:
        for k, v in rec["per_kernel"].items():
            out[k] = {"mfma_busy_of_busy_cus": v["mfma_busy_of_busy_cus"]}
    return out or None


PEAK_FP32_MATRIX_TFLOPS = 157.3  # dense fp32 MFMA, MI355X
PEAK_FP64_MATRIX_TFLOPS = 78.6   # dense fp64 MFMA, MI355X
PEAK_FP32_VECTOR_TFLOPS = 157.3  # fp32 vector, MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2 (packed) x 2 (FMA) x 2.4 GHz
R2D_KERNELS = ["k_damp_lambda", "k_damp_fill", "k_chol_panel", "k_chol_panel2", "k_gemm64", "k_gemm_ring64",
               "k_gemm_ring128", "k_make_u", "k_r2d_unit", "k_r2d_fill", "k_r2d_tile", "k_r2d_push", "k_r2d_obj"]


def bench_r2d(args, torch, Context, synth, dev):
    """Two-sided rounding (GPTQ-2D) of the square layer: target W / s on a
    signed 4-bit range, H = the layer's input Gram on the right, G = the Gram
    of a second seeded 4096-wide matrix on the left.  A step is both damped
    factors plus the rounding; the Grams are formed once before timing."""
    sq, og = synth.FULL["r2d"]
    print("# generating r2d inputs", file=sys.stderr, flush=True)
    lay = synth.layer(sq, dev)
    Xo = synth.calibration(og, dev)
    torch.cuda.synchronize()
    ctx = Context(dev)
    H = ctx.hessian(lay["X"])
    G = ctx.hessian(Xo)
    del Xo
    W = lay["W"]
    X2 = (W / (W.abs().max() / 7.5)).contiguous()
    m, n = X2.shape
    st = torch.cuda.current_stream(dev)

    def one_step(ev=None):
        if ev is not None:
            ev[0].record(st)
        UG, _, _ = ctx.factor(G, lam_rel=0.01)
        UH, _, _ = ctx.factor(H, lam_rel=0.01)
        if ev is not None:
            ev[1].record(st)
        r = ctx.round_2d(X2, UG, UH, -8, 7)
        if ev is not None:
            ev[2].record(st)
        return r

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    ctx.timing("k_r2d_push,k_r2d_tile")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    last = None
    for k in range(args.steps):
        last = one_step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    push_ms, push_n = ctx.kernel_time("k_r2d_push")
    tile_ms, tile_n = ctx.kernel_time("k_r2d_tile")
    ctx.timing("*")
    one_step()
    torch.cuda.synchronize()
    breakdown = {}
    for nm in R2D_KERNELS:
        ms, cnt = ctx.kernel_time(nm)
        if cnt:
            breakdown[nm] = {"ms": round(ms, 4), "launches": cnt}
    ctx.timing(None)
    ms_step = 1e3 * wall / args.steps
    fac = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    rnd = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    # algorithmic work of the pushes between tiles: every (tile, tile below)
    # and (tile, tile to the right) pair is one dense 64x64x64 product
    TM, TN = (m + 63) // 64, (n + 63) // 64
    pairs = sum((TM - I - 1) + (TN - J - 1) for I in range(TM) for J in range(TN))
    push_flops = pairs * 2 * 64 ** 3
    ach = push_flops * args.steps / (push_ms * 1e-3) / 1e12 if push_ms else 0.0
    # the in-tile walks: entry (k, l) of a tile pushes its delta down the
    # rows below it and its final C along the columns right of it, inside
    # the tile (2 flops per multiply-add), 2 * 64 * 2 * (0 + ... + 63) flops
    # per full tile; a launch walks the tiles of one anti-diagonal stage
    def tile_fl(mt, nt):
        return 2 * (nt * mt * (mt - 1) // 2 + mt * nt * (nt - 1) // 2)
    tile_flops = sum(tile_fl(min(64, m - 64 * I), min(64, n - 64 * J)) for I in range(TM) for J in range(TN))
    tile_launches = TM + TN - 1
    tile_avg_ms = tile_ms / max(tile_n, 1)
    tile_ach = tile_flops / tile_launches / (tile_avg_ms * 1e-3) / 1e12 if tile_n else 0.0
    line = {"metric": "ms per layer, two-sided rounding (GPTQ-2D) of a 4096x4096 layer", "value": round(ms_step, 4),
            "unit": "ms/layer", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic (seeded; the square layer and a second 4096-wide input)",
            "config": {"workload": "r2d: X = W/s [4096,4096] -> Z in [-8,7]; G from Y[65536,4096], "
                                   "H from X[262144,4096], lam 0.01 mean diag"},
            "stages_ms": {"factors": round(fac, 4), "round_2d": round(rnd, 4)},
            "kernels_one_step": breakdown,
            # the walk is a chain of 2 * 64 - 1 dependent steps per tile (each an
            # LDS read, the rounding, the pushes and a barrier), not limited by
            # any throughput: its fraction of the fp32 vector peak is small by
            # construction, and the per-step time is the figure that moves
            "roofline": {"kernel": "k_r2d_tile", "bound": "alu", "achieved": round(tile_ach, 4),
                         "peak": PEAK_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tile_ach / PEAK_FP32_VECTOR_TFLOPS, 6), "traffic": None,
                         "avg_launch_ms": round(tile_avg_ms, 4),
                         "flops_per_launch": tile_flops / tile_launches,
                         "latency": {"dependent_steps_per_launch": 2 * 64 - 1,
                                     "ns_per_step": round(tile_avg_ms * 1e6 / (2 * 64 - 1), 1),
                                     "launches_per_step": tile_n // max(args.steps, 1)}},
            "secondary": {"k_r2d_push": {"bound": "mfma", "achieved": round(ach, 2),
                                         "peak": PEAK_FP32_MATRIX_TFLOPS, "unit": "TFLOP/s",
                                         "frac": round(ach / PEAK_FP32_MATRIX_TFLOPS, 4),
                                         "avg_launch_ms": round(push_ms / max(push_n, 1), 4),
                                         "flops_per_step": push_flops}},
            "objective": {"J": last["J"]}}
    ctx.close()
    print(json.dumps(line), flush=True)


QR_KERNELS = ["k_syrk", "k_syrk_reduce", "k_damp_lambda", "k_damp_fill", "k_chol_panel2", "k_gemm_ring64",
              "k_gemm_ring128", "k_make_u", "k_qr_prep", "k_qr_out", "k_init_work", "k_sweep", "k_trail",
              "k_objective"]


def bench_qronos(args, torch, Context, synth, dev):
    """GPTQ with the quantised-input target on the square layer: Xq = X plus
    seeded noise (a stand-in for the inputs an already-quantised network
    feeds the layer).  A step is the whole call: Xq^T Xq and Xq^T X (one
    grouped SYRK launch), the factor, the target's three fp64 products and
    the sweep."""
    sq = synth.FULL["square"][0]
    print("# generating qronos inputs", file=sys.stderr, flush=True)
    lay = synth.layer(sq, dev)
    Xq = synth.perturbed(lay["X"], sq.seed)
    torch.cuda.synchronize()
    ctx = Context(dev)

    def one_step():
        return ctx.quantize_qronos(lay["W"], lay["X"], Xq, sq.bits, sq.group, sq.block, lam_rel=sq.lam_rel)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    ctx.timing("k_syrk")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    last = None
    for _ in range(args.steps):
        last = one_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    syrk_ms, syrk_n = ctx.kernel_time("k_syrk")
    ctx.timing("*")
    one_step()
    torch.cuda.synchronize()
    breakdown = {}
    for nm in QR_KERNELS:
        ms, cnt = ctx.kernel_time(nm)
        if cnt:
            breakdown[nm] = {"ms": round(ms, 4), "launches": cnt}
    ctx.timing(None)
    ms_step = 1e3 * wall / args.steps
    t, n = sq.tokens, sq.n
    flops = t * n * (n + 1) + 2 * t * n * n  # Xq^T Xq (triangle) + Xq^T X (full), one launch
    avg = syrk_ms / max(syrk_n, 1)
    ach = flops / (avg * 1e-3) / 1e12 if syrk_n else 0.0
    line = {"metric": "ms per layer, GPTQ with the quantised-input target, 4096x4096 4-bit g128",
            "value": round(ms_step, 4), "unit": "ms/layer", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; the square layer, Xq = bf16(X + 0.05 std(X) noise))",
            "config": {"workload": "qronos: W[4096,4096] X,Xq[262144,4096] 4-bit g128 B128"},
            "kernels_one_step": breakdown,
            "roofline": {"kernel": "k_syrk", "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                         "avg_launch_ms": round(avg, 4), "flops_per_launch": flops},
            "objective": {"J": last["J"], "J_lam": last["J_lam"]}}
    ctx.close()
    print(json.dumps(line), flush=True)


def bench_w4a16(args, torch, Context, synth, dev):
    """The W4A16 product of a deployed 4-bit square layer: Y = X What^T with X
    [8192, 4096] bf16 (the square layer's input recipe) and the stored form of
    a [4096, 4096] 4-bit g128 layer (seeded codes, scales, zero points), packed
    by the library before timing.  A step is one gptq_gemm_w4a16 call.  The
    w4a16_decode workload applies the same layer to 16 tokens (the few-row
    kernel), reported in microseconds against the HBM roof.  With --bits 2, 3
    or 8 the layer is stored at that width and the step is one
    gptq_gemm_wqa16 call (kernels k_gemm_wqa16 / k_gemv_wqa16)."""
    cfg = synth.W4A16
    M, N, K, group = cfg["M"], cfg["N"], cfg["K"], cfg["group"]
    decode = args.workload == "w4a16_decode"
    if decode:
        M = synth.W4A16_DECODE_M
    print("# generating w4a16 inputs", file=sys.stderr, flush=True)
    X = synth.w4a16_inputs(M, K, 92, dev)
    bits = args.bits
    if bits == 4:
        codes, scales, zeros = synth.w4_stored(N, K, group, 92)
    else:
        codes, scales, zeros = synth.wq_stored(N, K, group, bits, 92)
    ctx = Context(dev)
    P = ctx.pack_codes(codes.to(dev), bits)
    S, Z = scales.to(dev), zeros.to(dev)
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def one_step():
        if bits == 4:
            ctx.gemm_w4a16(X, P, S, Z, group, Y=Y)
        else:
            ctx.gemm_wqa16(X, P, S, Z, group, bits, Y=Y)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    wq = "w4a16" if bits == 4 else "wqa16"
    kname = ("k_gemv_" if decode else "k_gemm_") + wq
    ctx.timing(kname)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms, k_n = ctx.kernel_time(kname)
    ctx.timing(None)
    ms_step = 1e3 * wall / args.steps
    flops = 2.0 * M * N * K
    avg = k_ms / max(k_n, 1)
    ach = flops / (avg * 1e-3) / 1e12
    alg_bytes = M * K * 2 + N * K * bits // 8 + N * (K // group) * 5 + M * N * 4
    wname = "W%dA16" % bits
    label = "w4a16" if bits == 4 else "w%da16" % bits  # traffic records: profiles/<kernel>_<label>[_decode]_traffic.json
    if decode:
        gbs = alg_bytes / (avg * 1e-3) / 1e9
        line = {"metric": "us per %s product at decode size, X [%d, 4096] bf16, %d-bit g128 [4096, 4096]"
                          % (wname, M, bits),
                "value": round(ms_step * 1e3, 2), "unit": "us/product", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": False, "scaling": "weak",
                "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded; X from the square layer's input recipe, uniform %d-bit codes)" % bits,
                "config": {"workload": "w4a16_decode: X[%d,4096] bf16 x W[4096,4096] %d-bit g128 -> Y fp32"
                                       % (M, bits)},
                "roofline": {"kernel": kname, "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                             "traffic": kernel_traffic(kname, label + "_decode", "deploy.hip"),
                             "avg_launch_ms": round(avg, 5), "bytes_per_launch": alg_bytes}}
        ctx.close()
        print(json.dumps(line), flush=True)
        return
    line = {"metric": "TFLOP/s of the %s product Y = X What^T, X [8192, 4096] bf16, %d-bit g128 [4096, 4096]"
                      % (wname, bits),
            "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; X from the square layer's input recipe, uniform %d-bit codes)" % bits,
            "config": {"workload": "w4a16: X[8192,4096] bf16 x W[4096,4096] %d-bit g128 -> Y fp32" % bits},
            "roofline": {"kernel": kname, "bound": "mfma", "achieved": round(ach, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                         "traffic": kernel_traffic(kname, label, "deploy.hip"),
                         "avg_launch_ms": round(avg, 4), "flops_per_launch": flops,
                         "algorithmic_bytes_per_launch": alg_bytes}}
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle import gptq_ref as o
        rows = M  # the whole product (about 7 s on the host cores)
        Xs = synth.bits_to_numpy(X[:rows].cpu())
        c, sc, zf = codes.numpy(), scales.numpy(), zeros.numpy().astype(np.float32)
        t0 = time.perf_counter()
        o.gemm_w4a16(Xs, c, sc, zf, group, weight_bf16=True)
        t_s = time.perf_counter() - t0
        try:
            cores = len(os.sched_getaffinity(0))
        except Exception:
            cores = os.cpu_count()
        line["cpu_baseline"] = {"value": round(2.0 * rows * N * K / t_s / 1e12, 4), "unit": "TFLOP/s",
                                "cores": cores, "kind": "oracle",
                                "sample": "the float64 product on %d of %d rows of X (dequantisation "
                                          "included); measured %.2f s" % (rows, M, t_s)}
    ctx.close()
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="square",
                    choices=["square", "single", "lora", "lora_refine", "mlp", "vit", "r2d", "qronos", "w4a16",
                             "w4a16_decode"])
    ap.add_argument("--rounds", type=int, default=1, help="refinement rounds of the lora_refine workload")
    ap.add_argument("--bits", type=int, default=4, choices=[2, 3, 4, 8],
                    help="code width of the w4a16 and w4a16_decode workloads")
    ap.add_argument("--pipeline", choices=["batched", "separate"], default="batched",
                    help="square / single / mlp: one gptq_quantize_batched call per step (Hessian, factor and "
                         "sweep enqueued together, one host wait at the end), or one call per stage (the factor "
                         "waits for its pivot status before the sweep is enqueued)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (5 times), the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the pass runs on a single MI355X "
              "(--gpus %d is not supported)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from post_weight_quantization_gptq_amd import Context, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": 5}), flush=True)
        return
    if args.workload == "r2d":
        bench_r2d(args, torch, Context, synth, dev)
        return
    if args.workload == "qronos":
        bench_qronos(args, torch, Context, synth, dev)
        return
    if args.workload in ("w4a16", "w4a16_decode"):
        bench_w4a16(args, torch, Context, synth, dev)
        return
    specs = synth.FULL["lora" if args.workload == "lora_refine" else args.workload]
    print("# generating %s inputs" % args.workload, file=sys.stderr, flush=True)
    lays = [synth.layer(s, dev) for s in specs]
    torch.cuda.synchronize()
    ctx = Context(dev)
    st = torch.cuda.current_stream(dev)

    def one_step(evl=None):
        results = []
        if args.workload == "vit":
            layers = [dict(W=l["W"], X=l["X"], bits=s.bits, group=s.group, block=s.block, lam_rel=s.lam_rel)
                      for s, l in zip(specs, lays)]
            ctx.quantize_batched(layers)
            return layers
        shared = {}
        for li, (s, l) in enumerate(zip(specs, lays)):
            ev = evl[li] if evl is not None else None
            if s.kind == "lowrank":
                if args.workload == "lora_refine":
                    results.append(ctx.lora_refine(l["W"], l["X"], s.rank, s.bits, s.group, s.block,
                                                   rounds=args.rounds, lam_rel=s.lam_rel))
                else:
                    results.append(ctx.lora(l["W"], l["X"], s.rank, s.bits, s.group, s.block, lam_rel=s.lam_rel))
                continue
            if ev is not None:
                ev[0].record(st)
            if s.x_key and s.x_key in shared:
                # layers fed by the same input share one Hessian and its factor
                U, lam = shared[s.x_key]
                if ev is not None:
                    ev[1].record(st)
            else:
                H = ctx.hessian(l["X"])
                if ev is not None:
                    ev[1].record(st)
                U, info, lam = ctx.factor(H, lam_rel=s.lam_rel)
                if s.x_key:
                    shared[s.x_key] = (U, lam)
            if ev is not None:
                ev[2].record(st)
            r = ctx.quantize(l["W"], U, s.bits, s.group, s.block, lam)
            if ev is not None:
                ev[3].record(st)
            results.append(r)
        return results

    # the whole-layer entry: every stage of the step's layers enqueued at once;
    # layers fed by the same input pass it once and share its H and U
    blayers, firsts = [], {}
    for s, l in zip(specs, lays):
        d = dict(W=l["W"], bits=s.bits, group=s.group, block=s.block, lam_rel=s.lam_rel)
        if s.x_key and s.x_key in firsts:
            d["H"], d["U"] = firsts[s.x_key]["H"], firsts[s.x_key]["U"]
        else:
            d["X"] = l["X"]
            d["H"] = torch.empty((s.n, s.n), dtype=torch.float32, device=dev)
            d["U"] = torch.empty((s.n, s.n), dtype=torch.float32, device=dev)
            if s.x_key:
                firsts[s.x_key] = d
        blayers.append(d)
    batched = args.pipeline == "batched" and args.workload in ("square", "single", "mlp")

    def batched_step(evl=None):
        ctx.quantize_batched(blayers)
        return blayers

    step = batched_step if batched else one_step
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the Gram dominates every path: bf16 MFMA, or fp64 MFMA for the LoRA paths
    dominant = "k_syrk64" if args.workload in ("lora", "lora_refine") else "k_syrk"
    ctx.timing(dominant)
    stage = {"hessian": 0.0, "factor": 0.0, "quantize": 0.0}
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in specs] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    last = None
    for k in range(args.steps):
        last = step(evs[k] if args.workload in ("square", "single", "mlp") and not batched else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms, dom_launches = ctx.kernel_time(dominant)
    if batched:
        # stage times from separate calls with events between the stages (untimed steps)
        ctx.timing(None)
        for k in range(args.steps):
            one_step(evs[k])
        torch.cuda.synchronize()
    # per-kernel breakdown from one more (untimed) step with every launch bracketed
    ctx.timing("*")
    one_step()
    torch.cuda.synchronize()
    names = ["k_xpose", "k_syrk", "k_syrk_reduce", "k_syrk64", "k_syrk64_reduce", "k_damp_lambda", "k_damp_fill", "k_chol_panel", "k_chol_panel2",
             "k_gemm64", "k_gemm_ring64", "k_gemm_ring128", "k_make_u", "k_init_work", "k_rowfit", "k_sweep", "k_trail", "k_objective",
             "k_lora_lambda", "k_start_block", "k_dgemm", "k_dsum", "k_gram_chol", "k_apply", "k_lora_assemble",
             "k_lora_extract", "k_ref_init", "k_resid", "k_gfinal", "k_sum_parts", "k_f32_to_f64", "k_f64_to_f32",
             "k_olrc_out", "k_ritz", "k_ritz_resid", "k_ritz_conv", "k_cols"]
    breakdown = {}
    for nm in names:
        ms, cnt = ctx.kernel_time(nm)
        if cnt:
            breakdown[nm] = {"ms": round(ms, 4), "launches": cnt}
    ctx.timing(None)
    ms_step = 1e3 * wall / args.steps
    nlayers = len(specs)
    ms_layer = ms_step / nlayers

    fl, seen = [], set()
    for s in specs:
        f = layer_flops(s.out, s.n, s.tokens, s.block, s.n + s.rank)
        if s.x_key and s.x_key in seen:  # shared Hessian and factor: counted once
            f["total"] -= f["syrk"] + f["factor"]
            f["syrk"] = f["factor"] = 0
        seen.add(s.x_key)
        fl.append(f)
    total_flops = sum(f["total"] for f in fl)
    tflops = total_flops / (ms_step * 1e-3) / 1e12
    metric = METRIC if args.workload == "square" else (
        "ms per layer + TFLOP/s (frac of MFMA peak), GPTQ, %s workload (%d layers per step)" % (args.workload, len(specs)))
    line = {"metric": metric, "value": round(ms_layer, 4), "unit": "ms/layer", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded; shapes, spectra and outliers of the pages' layers)",
            "config": {"workload": "%s: %s" % (args.workload, ", ".join(
                "%s W[%d,%d] X[%d,%d] %d-bit g%d B%d" % (s.name, s.out, s.n, s.tokens, s.n, s.bits, s.group, s.block)
                for s in specs[:4]) + (" ... (%d layers)" % len(specs) if len(specs) > 4 else "")),
                       "pipeline": ("one gptq_quantize_batched call per step" if batched else
                                    "one call per stage")},
            "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "dtypes": "X bf16 -> H fp32 (bf16 MFMA, fp32 accumulate); factor fp64; sweep and trailing fp32"}
    if args.workload in ("square", "single", "mlp"):
        for k in range(args.steps):
            for e in evs[k]:
                stage["hessian"] += e[0].elapsed_time(e[1])
                stage["factor"] += e[1].elapsed_time(e[2])
                stage["quantize"] += e[2].elapsed_time(e[3])
        for key in stage:
            stage[key] = round(stage[key] / args.steps / nlayers, 4)
        line["stages_ms"] = stage
    line["kernels_one_step"] = breakdown
    if args.workload in ("square", "single", "mlp") and "k_trail" in breakdown and "k_sweep" in breakdown:
        # secondary rates from the breakdown step (event-bracketed kernel time,
        # wide updates overlapping the sweeps included): the trailing update
        # against the fp32 matrix roof, the sweep's bytes against HBM
        trail_fl = sum(f["trail"] for f in fl)
        sweep_bytes = sum(s.out * s.n * (4 + 4 + 1 + 4) + s.n * s.block * 4 for s in specs)  # W, W_orig, codes, E; U blocks
        t_tr = breakdown["k_trail"]["ms"] * 1e-3
        t_sw = breakdown["k_sweep"]["ms"] * 1e-3
        line["secondary"] = {
            "k_trail": {"tflops": round(trail_fl / t_tr / 1e12, 2), "peak": PEAK_FP32_MATRIX_TFLOPS,
                        "frac": round(trail_fl / t_tr / 1e12 / PEAK_FP32_MATRIX_TFLOPS, 4)},
            "k_sweep": {"gb_s": round(sweep_bytes / t_sw / 1e9, 1), "peak": PEAK_HBM_GBS,
                        "frac": round(sweep_bytes / t_sw / 1e9 / PEAK_HBM_GBS, 4), "bound": "latency"}}
    if "stages_ms" in line and line["stages_ms"]["factor"] > 0:
        # the factor stage (damping, Cholesky and inverse: 2 n^3 / 3 flops per
        # distinct Hessian) against the fp64 matrix roof, from the timed steps
        fac_fl = sum(f["factor"] for f in fl) / nlayers
        rate = fac_fl / (line["stages_ms"]["factor"] * 1e-3) / 1e12
        line.setdefault("secondary", {})["factor"] = {
            "tflops": round(rate, 2), "peak": PEAK_FP64_MATRIX_TFLOPS, "frac": round(rate / PEAK_FP64_MATRIX_TFLOPS, 4),
            "flops_per_layer": fac_fl}
    if dom_launches:
        # algorithmic flops of one launch (mean over the step's launches): the
        # triangle X^T X of every layer the launch covers
        per_launch = sum(f["syrk"] for f in fl) / dom_launches * args.steps
        avg_ms = dom_ms / dom_launches
        ach = per_launch / (avg_ms * 1e-3) / 1e12
        peak = PEAK_FP64_MATRIX_TFLOPS if dominant == "k_syrk64" else PEAK_BF16_TFLOPS
        line["roofline"] = {"kernel": dominant, "bound": "mfma", "achieved": round(ach, 2),
                            "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                            "traffic": syrk_traffic(args.workload) if dominant == "k_syrk" else None,
                            "avg_launch_ms": round(avg_ms, 4), "flops_per_launch": per_launch}
    if args.workload == "square":
        rates = counter_rates(args.workload)
        if rates:
            line["counters"] = rates
    if args.workload == "lora":
        line["objective"] = {"J": last[0]["J"], "J_lam": last[0]["J_lam"]}
    if args.workload == "lora_refine":
        line["objective"] = {"trace": last[0]["trace"], "rounds": args.rounds}
    if not args.no_cpu_baseline and args.workload in ("square", "single"):
        print("# timing the oracle on a host sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(specs[0], {"W": lays[0]["W"], "X": lays[0]["X"]})
    ctx.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Throughput of the FP4 block quantizer on one MI355X.

One step = one pass of the hot path over one batch: the global max pass and
the NVFP4 ScaleSweep (WMSE, window [-8, +7]) over a bf16 4096 x 4096 weight
with per-column importance, i.e. everything fp4q_quantize_nvfp4 does.

Prints ONE JSON line.  ``value`` is quantized elements per second (G/s) with
the inputs already resident in HBM; ten distinct input buffers (320 MiB, more
than the 256 MB Infinity Cache) are rotated so every step reads HBM.

The ``roofline`` object is for the dominant kernel (the sweep), timed alone
with HIP events on the stream it runs on (a call with a given global scale
launches exactly that kernel).  Its ``traffic`` is the calibrated
FETCH_SIZE + WRITE_SIZE bytes per launch recorded under profiles/ by
``python -m fp4_post_quantization_amd.evidence`` for the current kernel
sources, or null when the kernels changed since.  ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload on this host (one core on 2048 rows, and a
pool of forked processes over the whole matrix), before the GPU is
initialised.  Before the warmup steps,
untimed steps run for 0.3 s so the GPU has left its idle clocks.

Other workloads (for the design notes, not the headline line) are selected
with --config: c1, c2, c3a (MXFP4 AbsMax), c3b (MXFP4 window [-1,0]),
c3c (MXFP4 after 32-point Hadamard), c4 (8B layer, MSE then WMSE),
c5 (70B-shaped layer stream, 16-point Hadamard + WMSE; --layers N),
c5gate (one 70B-shaped gate projection, 16-point Hadamard + WMSE, repeated),
focus (FOCUS forward quantizer on the c2 weight, sub-blocks of 8),
study (AbsMax / ScaleSweep / exhaustive windows and MXFP4 code usage),
gptq (GPTQ with ScaleSweep group scales on the 4096 x 4096 weight),
w4a4 (an 8B-shaped decoder layer at 8192 tokens in W4A4 MXFP4: on-the-fly
activation quantization with a 32-point Hadamard, then the seven projections
on the scaled FP4 matrix cores against weights quantized in the same basis),
w4a4nv (the same layer with NVFP4 operands on the bf16 matrix cores),
oracle (the CPU oracle alone, one process, on a 256-row sample of each workload).
"""

import argparse
import json

import numpy as np
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# fp32 vector peak without packed-FP32 instructions (the library is compiled without them):
# 256 CU x 64 lanes x 2 flops (FMA) x 2.4 GHz = 78.6 TFLOP/s
VALU_PEAK_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12
METRIC = "G elements/s quantized (NVFP4 WMSE sweep) + % of MI355X HBM roofline"


def _alg_ops_per_element(n_cand, wmse, had=0):
    """Algorithmic fp32 operations per element: per candidate a scale
    multiply, E2M1 rounding, dequant multiply, subtract, square, [weight
    multiply] and one accumulate (an FMA counts as two); a Hadamard adds
    log2(n) butterflies + 1."""
    per_cand = 7 if wmse else 6
    return n_cand * per_cand + (int(math.log2(had)) + 1 if had else 0)


def _alg_bytes_per_element(in_bytes, block):
    # read x, write 4-bit codes, per block 1 B scale + 4 B loss + 1 B offset
    return in_bytes + 0.5 + 6.0 / block


def _events_time(fn, iters):
    import torch
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(iters):
        fn(i)
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def _rotating_copies(x, min_bytes=300 * 2**20, min_count=10):
    import torch
    nbytes = x.numel() * x.element_size()
    n = max(min_count, math.ceil(min_bytes / nbytes))
    if n * nbytes > 40 * 2**30:
        n = max(2, (40 * 2**30) // nbytes)
    bufs = [x]
    for _ in range(n - 1):
        bufs.append(torch.empty_like(x).copy_(x))
    return bufs


_POOL = {}


def _oracle_rows(bounds):
    """One worker of the all-cores CPU baseline: the oracle on rows [r0, r1)
    of the shared matrix with the whole matrix's global scale."""
    from oracle import quant as Q
    r0, r1 = bounds
    Q.quantize_nvfp4(_POOL["x"][r0:r1], _POOL["imp"], window=_POOL["window"], global_scale=_POOL["S"])
    return r1 - r0


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_cpu, imp, sample_rows, window=None):
    """The CPU oracle (numpy), unchanged, timed twice on this host: in one
    process (one core) on the first ``sample_rows`` rows, and as a pool of
    forked worker processes over row shards of the whole matrix (the
    workload's global scale computed once).  Runs before the GPU is touched
    (the pool forks)."""
    import multiprocessing as mp
    from oracle import quant as Q
    x = x_cpu.float().numpy()
    imp_np = None if imp is None else imp.numpy()
    xs = x[:sample_rows]
    t0 = time.perf_counter()
    Q.quantize_nvfp4(xs, imp_np, window=window)
    dt1 = time.perf_counter() - t0
    cores = min(16, len(os.sched_getaffinity(0)))
    _POOL.update(x=x, imp=imp_np, window=window)
    t0 = time.perf_counter()
    _POOL["S"] = Q.global_scale_nvfp4(x)
    rows = x.shape[0]
    bounds = [(rows * i // cores, rows * (i + 1) // cores) for i in range(cores)]
    with mp.get_context("fork").Pool(cores) as pool:
        done = sum(pool.map(_oracle_rows, bounds))
    dtp = time.perf_counter() - t0
    assert done == rows
    return {"value": x.size / dtp / 1e9, "unit": "G elements/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole {rows} x {x.shape[1]} workload in {cores} forked numpy processes (row shards, "
                      f"global scale computed once): {dtp:.1f} s",
            "single_core": {"value": xs.size / dt1 / 1e9, "cores": 1,
                            "sample": f"first {sample_rows} rows ({xs.size} elements), {dt1:.1f} s in one process"},
            "cpu_model": _cpu_model()}


def oracle_table(sample_rows=256):
    """The CPU oracle (numpy, unchanged) in one process on the first
    ``sample_rows`` rows of each workload: elements per second per config,
    for comparison with the GPU rates.  A sample's global scale is its own
    max/1536.  The 70B-shaped matrix is drawn on cuda:0 when a GPU is present
    (its defining generator), else on the CPU."""
    import torch
    import workloads as W
    from oracle import quant as Q
    dev = "cuda:0" if torch.cuda.is_available() else "cpu"
    x2, imp2 = W.c2_weight_and_importance()
    x3 = W.c3_activation()
    gate = W.c5_matrix(0, "gate", dev)[:sample_rows].float().cpu().numpy()
    f = lambda t, n=sample_rows: t[:n].float().numpy()
    cases = [
        ("c1 NVFP4 MSE fp32 256x1024 (whole)", lambda: Q.quantize_nvfp4(W.c1_weight().float().numpy()),
         256 * 1024),
        ("c2 NVFP4 WMSE [-8,7] bf16 4096x4096", lambda: Q.quantize_nvfp4(f(x2), imp2.numpy(), window=(-8, 7)),
         sample_rows * 4096),
        ("c3a MXFP4 AbsMax 8192x4096", lambda: Q.quantize_mxfp4(f(x3), window=(0, 0)), sample_rows * 4096),
        ("c3b MXFP4 [-1,0] 8192x4096", lambda: Q.quantize_mxfp4(f(x3), window=(-1, 0)), sample_rows * 4096),
        ("c3c MXFP4 [-1,0] after H32", lambda: Q.quantize_mxfp4(f(x3), window=(-1, 0), hadamard_n=32),
         sample_rows * 4096),
        ("c4 8B q projection, NVFP4 MSE [-3,7]", lambda: Q.quantize_nvfp4(f(W.c4_matrix("q"))), sample_rows * 4096),
        ("c4 8B q projection, NVFP4 WMSE [-8,7]",
         lambda: Q.quantize_nvfp4(f(W.c4_matrix("q")), W.c4_importance("q").numpy(), window=(-8, 7)),
         sample_rows * 4096),
        ("c5 70B gate layer 0, H16 + NVFP4 WMSE [-8,7]",
         lambda: Q.quantize_nvfp4(gate, W.c5_importance("gate").numpy(), window=(-8, 7), hadamard_n=16),
         sample_rows * 8192),
    ]
    out = []
    for name, fn, n in cases:
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        out.append({"config": name, "sample_elements": n, "seconds": round(dt, 3),
                    "G_elements_per_s": n / dt / 1e9})
        print(json.dumps(out[-1]), file=sys.stderr, flush=True)
    return {"config": "oracle", "cores": 1, "sample_rows": sample_rows, "cpu_model": _cpu_model(), "rows": out}


def prewarm(step, seconds=0.3):
    """Untimed steps for a fixed wall time before the warmup steps, so the
    GPU leaves its idle clock state before anything is timed."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step(i)
            i += 1
        torch.cuda.synchronize()


def bench_nvfp4_matrix(x, imp, window, had, steps, warmup):
    """Time the full call (max pass + sweep) and the sweep kernel alone."""
    import torch
    import fp4_post_quantization_amd as fq
    bufs = _rotating_copies(x)
    out = fq.quantize_nvfp4(bufs[0], imp, window=window, hadamard_n=had)
    ws = fq.workspace(x.device)
    fq.clear_status(ws)
    step = lambda i: fq.quantize_nvfp4(bufs[i % len(bufs)], imp, window=window, hadamard_n=had, out=out, ws=ws)
    prewarm(step)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = _events_time(step, steps)
    # per-step distribution (a second, separately timed pass: one event pair per step)
    per_step = []
    for i in range(steps):
        s_ev = torch.cuda.Event(enable_timing=True)
        e_ev = torch.cuda.Event(enable_timing=True)
        s_ev.record()
        step(i)
        e_ev.record()
        per_step.append((s_ev, e_ev))
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in per_step)
    pct = lambda q: us[min(len(us) - 1, int(q * (len(us) - 1) + 0.5))]
    bench_nvfp4_matrix.step_us = {"p10": round(pct(0.1), 2), "p50": round(pct(0.5), 2), "p90": round(pct(0.9), 2)}
    # out.global_scale now holds S; passing it back launches the sweep kernel only
    sweep = lambda i: fq.quantize_nvfp4(bufs[i % len(bufs)], imp, window=window, hadamard_n=had,
                                        global_scale=out.global_scale, out=out, ws=ws)
    for i in range(warmup):
        sweep(i)
    ms_sweep = _events_time(sweep, steps)
    torch.cuda.synchronize()
    status = fq.read_status(ws)
    if status:
        raise RuntimeError(f"device reported data error 0x{status:x}")
    return ms_step, ms_sweep


def run_c2(args, x_cpu, imp_cpu, cpu_line):
    x = x_cpu.to("cuda:0")
    imp = imp_cpu.to("cuda:0")
    rows, cols = x.shape
    n = rows * cols
    window = (-8, 7)
    ms_step, ms_sweep = bench_nvfp4_matrix(x, imp, window, 0, args.steps, args.warmup)
    value = n / (ms_step * 1e-3) / 1e9
    ops = _alg_ops_per_element(16, True)
    byts = _alg_bytes_per_element(2, 16)
    achieved_tflops = ops * n / (ms_sweep * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "G elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_us_percentiles": getattr(bench_nvfp4_matrix, "step_us", None),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "NVFP4 WMSE ScaleSweep, bf16 weight 4096x4096 (Student-t nu=4, std 0.02), "
                               "importance = Gram diagonal of 512x4096 lognormal-scaled activations, "
                               "block 16, E4M3 offsets [-8,+7]",
                   "rows": rows, "cols": cols, "input_dtype": "bf16", "block": 16, "window": list(window)},
        "hbm": {"alg_bytes_per_element": byts, "achieved_GBs": round(byts * n / (ms_step * 1e-3) / 1e9, 1),
                "peak_GBs": HBM_PEAK_GBS,
                "frac": round(byts * n / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"kernel": "nvfp4_sweep_kernel<bf16, WMSE, no rotation>", "bound": "alu",
                     "achieved": round(achieved_tflops, 3), "peak": round(VALU_PEAK_TFLOPS, 2),
                     "unit": "TFLOP/s", "frac": round(achieved_tflops / VALU_PEAK_TFLOPS, 4), "traffic": None,
                     "alg_ops_per_element": ops, "elements_per_launch": n,
                     "kernel_ms": round(ms_sweep, 5)},
    }
    from fp4_post_quantization_amd import evidence
    rec = evidence.committed_traffic("c2")
    if rec:  # calibrated FETCH_SIZE + WRITE_SIZE of this kernel source, from profiles/
        line["roofline"]["traffic"] = round(rec["traffic_bytes"])
    if cpu_line is not None:
        line["cpu_baseline"] = cpu_line
    return line


def run_other(args):
    """Side measurements for the design notes (not the headline)."""
    import torch
    import fp4_post_quantization_amd as fq
    import workloads as W
    res = {"config": args.config}
    if args.config == "c1":
        x = W.c1_weight().to("cuda:0")
        ms, msw = bench_nvfp4_matrix(x, None, (-3, 7), 0, args.steps, args.warmup)
        res.update(elements=x.numel(), ms_step=ms, ms_sweep=msw, gel_s=x.numel() / ms / 1e6)
    elif args.config.startswith("c3"):
        x = W.c3_activation().to("cuda:0")
        window = (0, 0) if args.config == "c3a" else (-1, 0)
        had = 32 if args.config == "c3c" else 0
        bufs = _rotating_copies(x)
        out = fq.quantize_mxfp4(bufs[0], window=window, hadamard_n=had)
        step = lambda i: fq.quantize_mxfp4(bufs[i % len(bufs)], window=window, hadamard_n=had, out=out)
        prewarm(step)
        for i in range(args.warmup):
            step(i)
        ms = _events_time(step, args.steps)
        byts = _alg_bytes_per_element(2, 32)
        res.update(elements=x.numel(), ms_step=ms, gel_s=x.numel() / ms / 1e6,
                   hbm_GBs=byts * x.numel() / ms / 1e6, hbm_frac=byts * x.numel() / ms / 1e6 / HBM_PEAK_GBS)
    elif args.config == "focus":
        # FOCUS forward quantizer on the c2 weight: stored scales from the
        # sweep, FP16 coefficients per 8-element sub-block, dequantized output
        x, imp = W.c2_weight_and_importance()
        x = x.to("cuda:0")
        base = fq.quantize_nvfp4(x, imp.to("cuda:0"))
        c = torch.exp(0.1 * torch.randn(x.shape[0], x.shape[1] // 8, device="cuda:0")).to(torch.float16)
        bufs = _rotating_copies(x)
        codes, dq = fq.quantize_relaxed(bufs[0], base.scales, c, global_scale=base.global_scale, sub=8)
        step = lambda i: fq.quantize_relaxed(bufs[i % len(bufs)], base.scales, c, global_scale=base.global_scale,
                                             sub=8, out_codes=codes, out_dequant=dq)
        prewarm(step)
        for i in range(args.warmup):
            step(i)
        ms = _events_time(step, args.steps)
        byts = 2 + 2 / 8 + 1 / 16 + 0.5 + 4  # x, coefficients, scales in; codes, dequantized out
        res.update(elements=x.numel(), ms_step=ms, gel_s=x.numel() / ms / 1e6,
                   hbm_GBs=byts * x.numel() / ms / 1e6, hbm_frac=byts * x.numel() / ms / 1e6 / HBM_PEAK_GBS)
    elif args.config == "study":
        # AbsMax vs ScaleSweep vs exhaustive windows; MXFP4 code usage
        from fp4_post_quantization_amd import study
        x2, imp2 = W.c2_weight_and_importance()
        res["c2_wmse"] = study.nvfp4_scale_rules(x2.to("cuda:0"), imp2.to("cuda:0"))
        res["c4_q_mse"] = study.nvfp4_scale_rules(W.c4_matrix("q").to("cuda:0"))
        res["c1_mse"] = study.nvfp4_scale_rules(W.c1_weight().to("cuda:0"))
        res["c5_gate_h16_wmse"] = study.nvfp4_scale_rules(W.c5_matrix(0, "gate", "cuda:0"),
                                                          W.c5_importance("gate").to("cuda:0"), iters=5,
                                                          hadamard_n=16)
        x3 = W.c3_activation().to("cuda:0")
        res["c3_mxfp4"] = [study.mxfp4_code_usage(x3, window=w, hadamard_n=h)
                           for h in (0, 32) for w in ((0, 0), (-1, 0))]
    elif args.config == "gptq":
        # GPTQ with ScaleSweep group scales on the 4096 x 4096 c2 weight,
        # Hessian from 2048 correlated synthetic calibration tokens
        x, imp = W.c2_weight_and_importance()
        X = W.calibration_activations(2048, 4096, seed=204)
        H, U = W.hessian_and_factor(X)
        xd = x.to("cuda:0").float()
        Ud = torch.from_numpy(U).to("cuda:0")
        Hd = torch.from_numpy(H).to("cuda:0")
        impd = torch.from_numpy(np.diag(H).astype(np.float32)).to("cuda:0")

        def proxy(codes, scales, S):
            xh = fq.dequantize("nvfp4", codes, scales, S).double()
            d = xd.double() - xh
            return float(((d @ Hd) * d).sum())

        for name, im in (("mse", None), ("wmse", impd)):
            r = fq.gptq_nvfp4(xd, Ud, im, check=True)
            step = lambda i: fq.gptq_nvfp4(xd, Ud, im)
            prewarm(step, seconds=0.5)
            ms = _events_time(step, max(3, args.steps // 10))
            rtn = fq.quantize_nvfp4(xd, im)
            ab = fq.quantize_nvfp4(xd, im, window=(0, 0))
            res[name] = {"ms": ms, "gel_s": xd.numel() / ms / 1e6,
                         "proxy_gptq": proxy(r.codes, r.scales, r.global_scale),
                         "proxy_rtn_sweep": proxy(rtn.codes, rtn.scales, rtn.global_scale),
                         "proxy_rtn_absmax": proxy(ab.codes, ab.scales, ab.global_scale)}

        def proxy_mx(codes, scales):
            xh = fq.dequantize("mxfp4", codes, scales).double()
            d = xd.double() - xh
            return float(((d @ Hd) * d).sum())

        # MXFP4 group scales (E8M0, window [-1, 0]); the same weight and Hessian
        for name, im in (("mxfp4_mse", None), ("mxfp4_wmse", impd)):
            r = fq.gptq_mxfp4(xd, Ud, im, check=True)
            step = lambda i: fq.gptq_mxfp4(xd, Ud, im)
            prewarm(step, seconds=0.5)
            ms = _events_time(step, max(3, args.steps // 10))
            rtn = fq.quantize_mxfp4(xd, im)
            ab = fq.quantize_mxfp4(xd, im, window=(0, 0))
            res[name] = {"ms": ms, "gel_s": xd.numel() / ms / 1e6,
                         "proxy_gptq": proxy_mx(r.codes, r.scales),
                         "proxy_rtn_sweep": proxy_mx(rtn.codes, rtn.scales),
                         "proxy_rtn_absmax": proxy_mx(ab.codes, ab.scales)}
    elif args.config == "c4":
        total_ms = {"mse": 0.0, "wmse": 0.0}
        n = 0
        for name in W.LAYER_8B:
            x = W.c4_matrix(name).to("cuda:0")
            imp = W.c4_importance(name).to("cuda:0")
            n += x.numel()
            for loss, im, win in (("mse", None, (-3, 7)), ("wmse", imp, (-8, 7))):
                ms, _ = bench_nvfp4_matrix(x, im, win, 0, max(3, args.steps // 5), 2)
                total_ms[loss] += ms
            del x
            torch.cuda.empty_cache()
        res.update(elements=n, ms_layer=total_ms, gel_s={k: n / v / 1e6 for k, v in total_ms.items()})
    elif args.config == "c5gate":
        # one 70B-shaped gate projection (28672 x 8192, 470 MB bf16) with H16 + WMSE, repeated: the c5
        # kernel on a single shape (the c5 stream mixes seven)
        x = W.c5_matrix(0, "gate", "cuda:0")
        imp = W.c5_importance("gate").to("cuda:0")
        out = fq.quantize_nvfp4(x, imp, hadamard_n=16, check=True)
        step = lambda i: fq.quantize_nvfp4(x, imp, hadamard_n=16, out=out)
        prewarm(step)
        for i in range(args.warmup):
            step(i)
        ms = _events_time(step, args.steps)
        res.update(elements=x.numel(), ms_step=ms, gel_s=x.numel() / ms / 1e6)
    elif args.config == "c5":
        imps = {name: W.c5_importance(name).to("cuda:0") for name in W.LAYER_70B}
        warm = W.c5_matrix(0, "k", "cuda:0")
        prewarm(lambda i: fq.quantize_nvfp4(warm, imps["k"], hadamard_n=16))
        del warm
        out_ms = 0.0
        n = 0
        for layer in range(args.layers):
            for name in W.LAYER_70B:
                x = W.c5_matrix(layer, name, "cuda:0")
                torch.cuda.synchronize()
                s = torch.cuda.Event(enable_timing=True)
                e = torch.cuda.Event(enable_timing=True)
                s.record()
                fq.quantize_nvfp4(x, imps[name], hadamard_n=16)
                e.record()
                e.synchronize()
                out_ms += s.elapsed_time(e)
                n += x.numel()
                del x
            print(f"layer {layer} done, {n / out_ms / 1e6:.1f} G el/s so far", file=sys.stderr, flush=True)
        res.update(layers=args.layers, elements=n, ms_total=out_ms, gel_s=n / out_ms / 1e6)
    elif args.config == "w4a4":
        res.update(run_w4a4(args))
    elif args.config == "w4a4nv":
        res.update(run_w4a4(args, fmt="nvfp4"))
    else:
        raise SystemExit(f"unknown config {args.config}")
    return res


def run_w4a4(args, fmt="mxfp4"):
    """8B-shaped layer in W4A4 at 8192 tokens: per layer step, the four
    activation inputs are quantized and the seven projections run as FP4
    GEMMs (bf16 out) against weights quantized offline.  MXFP4: AbsMax
    activations with a fused 32-point Hadamard, weights in the same rotated
    basis with window [-1, 0], scaled-FP4 matrix cores.  NVFP4: AbsMax
    activations, weights by the MSE sweep [-3, +7], operands decoded to bf16
    for the bf16 matrix cores."""
    import torch
    import fp4_post_quantization_amd as fq
    import workloads as W
    dev = "cuda:0"
    mx = fmt == "mxfp4"
    acts = {n: W.w4a4_activation(n, dev) for n in W.W4A4_INPUTS}

    def quant_act(x, out=None, check=False):
        if mx:
            return fq.quantize_mxfp4(x, window=(0, 0), hadamard_n=32, out=out, with_loss=False, check=check)
        return fq.quantize_nvfp4(x, window=(0, 0), out=out, with_loss=False, check=check)

    lib = fq._lib.load()
    ws_bytes = lib.fp4q_gemm_mxfp4_workspace_bytes if mx else lib.fp4q_gemm_nvfp4_workspace_bytes
    ws = torch.empty(max(max(ws_bytes(W.W4A4_TOKENS, n, k) for n, k in W.LAYER_8B.values()), 16),
                     dtype=torch.uint8, device=dev)

    def gemm(a, b, out=None, out_dtype=torch.bfloat16):
        if mx:
            return fq.gemm_mxfp4(a, b, out=out, out_dtype=out_dtype, workspace_buf=ws)
        return fq.gemm_nvfp4(a, b, out=out, out_dtype=out_dtype, workspace_buf=ws)

    wq, flops, err = {}, {}, {}
    for name in W.LAYER_8B:
        w = W.c4_matrix(name).to(dev)
        if mx:
            wq[name] = fq.quantize_mxfp4(w, window=(-1, 0), hadamard_n=32, with_loss=False, check=True)
        else:
            wq[name] = fq.quantize_nvfp4(w, window=(-3, 7), with_loss=False, check=True)
        flops[name] = 2 * W.W4A4_TOKENS * w.shape[0] * w.shape[1]
        # accuracy of the W4A4 product on 256 sampled tokens against the unquantized product
        xs = acts[W.W4A4_READS[name]][:256]
        c = gemm(quant_act(xs), wq[name], out_dtype=torch.float32)
        ref = xs.float() @ w.float().t()
        err[name] = float((c - ref).norm() / ref.norm())
        del w
    aq = {n: quant_act(x, check=True) for n, x in acts.items()}
    outs = {n: torch.empty((W.W4A4_TOKENS, wq[n].codes.shape[0]), dtype=torch.bfloat16, device=dev)
            for n in W.LAYER_8B}

    def quant_step():
        for n, x in acts.items():
            quant_act(x, out=aq[n])

    def gemm_step():
        for n in W.LAYER_8B:
            gemm(aq[W.W4A4_READS[n]], wq[n], out=outs[n])

    def layer(i):
        quant_step()
        gemm_step()

    prewarm(layer, seconds=0.5)
    for i in range(args.warmup):
        layer(i)
    ms_layer = _events_time(layer, args.steps)
    ms_quant = _events_time(lambda i: quant_step(), args.steps)
    ms_gemm = _events_time(lambda i: gemm_step(), args.steps)
    per = {}
    for n in W.LAYER_8B:
        ms_n = _events_time(lambda i, n=n: gemm(aq[W.W4A4_READS[n]], wq[n], out=outs[n]), args.steps)
        per[n] = {"shape_mnk": [W.W4A4_TOKENS, *W.LAYER_8B[n]], "ms": ms_n,
                  "tflops": flops[n] / ms_n / 1e9, "rel_err_vs_unquantized": err[n]}
    total_flops = sum(flops.values())
    return {"format": fmt, "tokens": W.W4A4_TOKENS, "ms_layer": ms_layer, "ms_activation_quant": ms_quant, "ms_gemms": ms_gemm,
            "gemm_tflops": total_flops / ms_gemm / 1e9, "layer_tflops": total_flops / ms_layer / 1e9,
            "matrix_core_dense_peak_tflops": 10100.0 if mx else 2500.0, "per_matrix": per}


def copy_calibration(nbytes=256 * 2**20, reps=3):
    """A kernel of known traffic (reads and writes nbytes once each) whose HBM
    counters calibrate FETCH_SIZE / WRITE_SIZE of the quantizer's kernels.  An
    int32 bitwise NOT: an elementwise kernel no workload runs itself, so its
    counters are found by name."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--layers", type=int, default=2)
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 256 MiB read + 256 MiB write elementwise kernel (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this quantizer runs on a single MI355X "
              "(no sharding or collectives are built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    cpu_line = None
    if args.config == "c2":
        import workloads as W
        x_cpu, imp_cpu = W.c2_weight_and_importance()
        if not args.no_cpu_baseline:  # before the GPU is initialised: the CPU baseline forks
            cpu_line = cpu_baseline(x_cpu, imp_cpu, args.cpu_rows, window=(-8, 7))
    if args.config == "oracle":  # the oracle's own host rates, no GPU work
        print(json.dumps(oracle_table()), flush=True)
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    line = run_c2(args, x_cpu, imp_cpu, cpu_line) if args.config == "c2" else run_other(args)
    if args.copy_calib:
        copy_calibration()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

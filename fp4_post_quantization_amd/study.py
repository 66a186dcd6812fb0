"""Scale-search study on the quantizer kernels.

Three NVFP4 scale rules run on the same kernel by changing only the window
of E4M3 bit-pattern offsets ("Resumo Técnico: ScaleSweep"):
  * AbsMax round-to-nearest: window (0, 0) (Declaração do Problema names
    AbsMax as the current initialization that leaves a gap to the optimum);
  * ScaleSweep: (-3, +7) for MSE, (-8, +7) for WMSE (2. Limites Teóricos,
    3. Implementação: overhead claimed negligible);
  * exhaustive: (-126, +126), every positive finite E4M3 scale (2.: called
    computationally inefficient).
For each the study reports the step time and the per-block losses; the gap
AbsMax - sweep is what the search gains, sweep - exhaustive what the window
gives up.

For MXFP4 activations it reports the code-usage statistics of "Resumo
Técnico: TORQ" (1. Declaração do Problema): the share of zero codes in the
blocks with the largest maxima, and "code collapse", the share of elements
whose code lies in the upper half of the E2M1 magnitude range, unrotated and
after a block Hadamard rotation ("Bridging the Gap ... Microscaling FP4",
2. Metodologia: rotation spreads outliers).

Counting runs on the GPU with torch reductions over the kernels' outputs.
"""

import torch

from . import quantize_mxfp4, quantize_nvfp4

WINDOWS = {"absmax": (0, 0), "exhaustive": (-126, 126)}


def code_histogram(codes):
    """Counts of the 16 four-bit codes in a packed code tensor (int64 [16])."""
    c = codes.reshape(-1)
    lo = (c & 0xF).to(torch.int64)
    hi = (c >> 4).to(torch.int64)
    return torch.bincount(lo, minlength=16) + torch.bincount(hi, minlength=16)


def magnitude_histogram(codes):
    """Counts of the 8 E2M1 magnitudes (sign folded), int64 [8]."""
    h = code_histogram(codes)
    return h[:8] + h[8:]


def _events_ms(fn, iters):
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


QUANTILES = (0.5, 0.9, 0.99)


def quantiles(v):
    """p50 / p90 / p99 / max of a 1-D tensor (sorted on the device; no size
    limit), as floats."""
    v = v.reshape(-1).double().sort().values
    n = v.numel()
    out = {f"p{int(round(q * 100))}": float(v[min(n - 1, int(q * (n - 1) + 0.5))]) for q in QUANTILES}
    out["max"] = float(v[-1])
    return out


def gap_quantiles(l_from, l_to):
    """Per-block gap l_from - l_to (never negative here: the narrower rule's
    candidates are a subset) and the same gap relative to l_from, as
    quantiles over the blocks (blocks with l_from = 0 have relative gap 0)."""
    g = (l_from - l_to).reshape(-1)
    rel = torch.where(l_from.reshape(-1) > 0, g / l_from.reshape(-1), torch.zeros_like(g))
    return {"absolute": quantiles(g), "relative": quantiles(rel), "negative_blocks": int((g < 0).sum())}


def nvfp4_block_losses(x, importance=None, hadamard_n=0):
    """Per-block losses (float64) of AbsMax, the ScaleSweep window and the
    exhaustive window on one matrix, no timing."""
    sweep_window = (-8, 7) if importance is not None else (-3, 7)
    rules = {"absmax": (0, 0), "sweep": sweep_window, "exhaustive": (-126, 126)}
    return {k: quantize_nvfp4(x, importance, window=w, hadamard_n=hadamard_n, check=True).block_loss.double()
            for k, w in rules.items()}


def gap_report(losses):
    """Gap quantiles AbsMax - sweep and sweep - exhaustive over the blocks of
    one or several matrices (lists of per-block loss tensors are pooled)."""
    cat = {k: torch.cat([v.reshape(-1) for v in (vs if isinstance(vs, list) else [vs])])
           for k, vs in losses.items()}
    a, s, e = cat["absmax"], cat["sweep"], cat["exhaustive"]
    return {"blocks": a.numel(),
            "absmax_minus_sweep": gap_quantiles(a, s),
            "sweep_minus_exhaustive": gap_quantiles(s, e),
            "loss_reduction_sweep_vs_absmax": 1 - float(s.sum() / a.sum()),
            "loss_reduction_exhaustive_vs_sweep": 1 - float(e.sum() / s.sum()) if float(s.sum()) else 0.0,
            "blocks_where_exhaustive_beats_sweep": float((e < s).double().mean())}


def mxfp4_block_losses(x, importance=None, hadamard_n=0, window=(-1, 0)):
    """Per-block MXFP4 losses for AbsMax (0, 0), the exponent window, and the
    widest window the call takes (-16, +16: a block whose best exponent lies
    16 binades below its maximum's would zero every element)."""
    rules = {"absmax": (0, 0), "sweep": window, "exhaustive": (-16, 16)}
    return {k: quantize_mxfp4(x, importance, window=w, hadamard_n=hadamard_n, check=True).block_loss.double()
            for k, w in rules.items()}


def nvfp4_scale_rules(x, importance=None, iters=20, hadamard_n=0):
    """AbsMax vs ScaleSweep vs exhaustive on one matrix (after the optional block rotation)."""
    sweep_window = (-8, 7) if importance is not None else (-3, 7)
    rules = {"absmax": (0, 0), "sweep": sweep_window, "exhaustive": (-126, 126)}
    res = {}
    out = {}
    for name, win in rules.items():
        r = quantize_nvfp4(x, importance, window=win, hadamard_n=hadamard_n, check=True)
        out[name] = r
        ms = _events_ms(lambda: quantize_nvfp4(x, importance, window=win, hadamard_n=hadamard_n, out=r), iters)
        res[name] = {"window": list(win), "ms": ms, "loss_sum": float(r.block_loss.double().sum())}
    a, s, e = (out[k].block_loss.double() for k in ("absmax", "sweep", "exhaustive"))
    res["gaps"] = gap_report({"absmax": a, "sweep": s, "exhaustive": e})
    nblk = a.numel()
    res["blocks"] = nblk
    res["sweep_vs_absmax"] = {
        "loss_reduction": 1 - res["sweep"]["loss_sum"] / res["absmax"]["loss_sum"],
        "blocks_improved": float((s < a).double().mean()),
        "blocks_worse": float((s > a).double().mean()),
        "time_ratio": res["sweep"]["ms"] / res["absmax"]["ms"],
    }
    res["exhaustive_vs_sweep"] = {
        "loss_reduction": 1 - res["exhaustive"]["loss_sum"] / res["sweep"]["loss_sum"],
        "blocks_improved": float((e < s).double().mean()),
        "blocks_worse": float((e > s).double().mean()),
        "time_ratio": res["exhaustive"]["ms"] / res["sweep"]["ms"],
    }
    off = out["sweep"].offsets.to(torch.int64).reshape(-1) - sweep_window[0]
    res["sweep_offset_histogram"] = {str(i + sweep_window[0]): int(v)
                                     for i, v in enumerate(torch.bincount(off, minlength=sweep_window[1] - sweep_window[0] + 1).tolist())}
    offx = out["exhaustive"].offsets.to(torch.int64).reshape(-1)
    res["exhaustive_outside_window"] = float(((offx < sweep_window[0]) | (offx > sweep_window[1])).double().mean())
    return res


def mxfp4_code_usage(x, window=(0, 0), hadamard_n=0, top_frac=0.01):
    """TORQ's code-usage statistics for one MXFP4 quantization."""
    r = quantize_mxfp4(x, window=window, hadamard_n=hadamard_n, check=True)
    rows, half = r.codes.shape
    mags = magnitude_histogram(r.codes).double()
    total = float(mags.sum())
    # per-block zero fraction for the blocks with the largest scales
    c = r.codes.reshape(rows, half // 16, 16)
    nib = torch.stack([c & 0xF, c >> 4], dim=-1).reshape(rows, half // 16, 32)
    zero = ((nib & 7) == 0).double().mean(-1).reshape(-1)
    sc = r.scales.reshape(-1).to(torch.int64)
    k = max(1, int(top_frac * sc.numel()))
    top = torch.topk(sc.double() + 1e-9 * torch.arange(sc.numel(), device=sc.device), k).indices
    return {
        "window": list(window),
        "hadamard_n": hadamard_n,
        "zero_code_fraction": float(mags[0] / total),
        "upper_half_code_fraction": float(mags[4:].sum() / total),
        "magnitude_histogram": [int(v) for v in mags.tolist()],
        "zero_fraction_in_top_blocks": float(zero[top].mean()),
        "top_blocks": k,
        "loss_sum": float(r.block_loss.double().sum()),
        "x_energy": float(x.double().pow(2).sum()),
    }

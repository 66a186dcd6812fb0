"""Float64 tools for checking the scale-search bounds (oracle; test
infrastructure).

"Resumo Técnico: ScaleSweep", 2. Limites Teóricos para Varredura Eficiente:
  * Lemma 4.1 -- a block scale s above 12/7 of the AbsMax base never gives a
    smaller loss than s/2, so the sweep stops at bit-pattern offset +7;
  * Lemma 4.3 -- for MSE the optimal scale is at least 4/5 of the base
    (offset -3);
  * for WMSE the lower end 1/2 of the base (offset -8) is set empirically.
These functions evaluate losses in float64 with the E2M1 decision taken on
the float64 quotient u / V, independently of the float32 canonical path.
"""

import numpy as np

from . import formats as F


def e2m1_nearest64(y):
    """E2M1 magnitude nearest to y >= 0 in float64 by direct distance search
    over the eight magnitudes; ties go to the even code index."""
    # every y above 6 has 6 as its nearest magnitude; capping at 7 keeps the
    # float64 distances exact for huge y
    y = np.minimum(np.asarray(y, dtype=np.float64), 7.0)
    grid = F.E2M1_VALUES.astype(np.float64)
    dist = np.abs(y[..., None] - grid)
    best = dist.min(axis=-1, keepdims=True)
    hit = dist == best
    # among equidistant magnitudes prefer an even index
    even_hit = hit & (np.arange(8) % 2 == 0)
    idx = np.where(even_hit.any(axis=-1), np.argmax(even_hit, axis=-1), np.argmax(hit, axis=-1))
    return grid[idx]


def block_loss64(u, V, w=None):
    """sum_i w_i (u_i - V * Q(u_i / V))**2 in float64 for each candidate V.

    u: [..., B] magnitudes (float64); V: [..., K] candidate scales; returns
    [..., K]."""
    u = np.asarray(u, dtype=np.float64)[..., None, :]
    V = np.asarray(V, dtype=np.float64)[..., :, None]
    q = e2m1_nearest64(u / V)
    err = (u - q * V) ** 2
    if w is not None:
        err = err * np.asarray(w, dtype=np.float64)[..., None, :]
    return err.sum(axis=-1)


def exhaustive_best_pattern64(u, w=None):
    """Pattern (1..126) minimizing the float64 loss over all 126 positive
    finite E4M3 scales; ties go to the smaller pattern."""
    V = F.E4M3_VALUES64[1:]
    L = block_loss64(u, np.broadcast_to(V, np.shape(u)[:-1] + V.shape), w)
    return 1 + np.argmin(L, axis=-1), L


def pattern_window_envelope(lo_factor, hi_factor):
    """For every normal base pattern b (0x08..0x77) and every t whose
    nearest E4M3 pattern is b, collect the patterns p with
    lo_factor * t <= V[p] <= hi_factor * t; return the smallest and largest
    offset p - b seen.  Each preimage interval is sampled at its two ends
    (open ends approached by one float32 step) and 199 interior points."""
    vals = F.E4M3_VALUES64
    mids = (vals[:-1] + vals[1:]) / 2
    lo_off, hi_off = 0, 0
    for b in range(0x08, 0x78):
        t_lo, t_hi = mids[b - 1], mids[b]
        ts = np.linspace(t_lo, t_hi, 201)
        ts[0] = np.nextafter(np.float32(t_lo), np.float32(np.inf))
        ts[-1] = np.nextafter(np.float32(t_hi), np.float32(0))
        ts = ts.astype(np.float32).astype(np.float64)
        for t in ts:
            ok = np.nonzero((vals >= lo_factor * t) & (vals <= hi_factor * t))[0]
            ok = ok[ok >= 1]
            if ok.size:
                lo_off = min(lo_off, int(ok.min()) - b)
                hi_off = max(hi_off, int(ok.max()) - b)
    return lo_off, hi_off

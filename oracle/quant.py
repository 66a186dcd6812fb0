"""NVFP4 ScaleSweep and MXFP4 exponent sweep (oracle; test infrastructure).

Layout: x is a row-major R x C matrix; blocks are contiguous runs of
``block`` columns inside a row (16 for NVFP4, 32 for MXFP4 -- "FOCUS: FP4
Optimization via Coupled-Relaxation and Dual-Granularity Scaling",
Declaração do Problema and 3. Escalonamento de Dupla Granularidade).

Every float32 step is one IEEE-754 round-to-nearest-even operation on numpy
float32 arrays, in the order written below.

NVFP4 ("Resumo Técnico: ScaleSweep")
  1. Global scale (2. Limites Teóricos, Escala Global):
       amax = max |x| over the tensor;  S = fp32(amax / 1536)  (1536 = 256 * 6);
       S_inv = fp32(1 / S), or 0 when S = 0.
  2. u = fp32(|x| * S_inv): magnitudes in units of S.
  3. AbsMax base scale s_base (Lemma 4.1 names it the block maximum rounded to
     FP8): a_b = max over the block of u; t_b = fp32(a_b / 6);
     base = max(RNE_E4M3(t_b), 1) as a bit pattern.  Dividing by 6 (the
     largest E2M1 magnitude) makes the block maximum land on the top code; it
     is the reading under which the page's bit-pattern offsets +7 / -3 / -8
     are exactly the envelopes of 12/7, 4/5 and 1/2 times the base scale.
  4. Candidates (2. Limites Teóricos and 3. Implementação): the E4M3 patterns
     p = base + o for o in [lo, hi] (default [-3, 7] for MSE, [-8, 7] for
     WMSE), clipped to 1..126.
  5. Per candidate, with V = E4M3 value of p and R = fp32(1/V):
       y = fp32(u * R); q = RNE_E2M1(y); d = q * V (exact); e = fp32(u - d);
       L_p = the block's squared errors summed in element order, each term
       added with a single rounding: acc <- fp32(t_i * e_i + acc) (a fused
       multiply-add), acc starting at 0, with t_i = e_i for MSE and
       t_i = fp32(w_col * e_i) for WMSE (importance of the element's column,
       1. Objetivos de Otimização).
  6. p* = smallest p whose L_p is the minimum over the candidates.
  7. Outputs: scale byte p*; code = (signbit(x) << 3) | index(q at p*);
     offset = p* - base; block loss = fp32(L_{p*} * fp32(S * S)); S.

MXFP4 ("Bridging the Gap ... Microscaling FP4", 2. Metodologia, MSE-optimised
grid; "Resumo Técnico: TORQ", B. Rotação de Alinhamento Micro, S-step)
  u = |x|; a_b = block max; E_base = min{E integer : 6 * 2**E >= a_b}, clamped
  to [-127, 127] (a_b = 0 gives -127): the block maximum maps onto the largest
  code without clipping.  Candidates E in [E_base + lo, E_base + hi] clipped to
  [-127, 127] (default lo, hi = -1, 0); per E: y = fp32(u * 2**-E);
  q = RNE_E2M1(y); d = q * 2**E (exact); e as above; L = the fused in-order
  sum above over all 32 elements of the block (one rounding per term, the
  same rule as the NVFP4 block's 16).
  E* = smallest E with the minimum loss.  Scale byte E* + 127, offset
  E* - E_base, loss L_{E*} (no global scale).
"""

from dataclasses import dataclass

import numpy as np

from . import formats as F
from .hadamard import block_hadamard


def fma_f32(a, b, c):
    """fp32(a * b + c) rounded once (to nearest, ties to even), for float32
    inputs, computed exactly in float64: a * b is exact there (two 24-bit
    significands); s = fp64(a*b + c) carries an exact error err (Knuth's
    two-sum), and rounding s to float32 is only wrong when s lies exactly
    half-way between two float32 values while err is not zero; then the
    sign of err picks the side."""
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    b64 = np.asarray(b, dtype=np.float32).astype(np.float64)
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a64 * b64
    s = p + c64
    bv = s - p
    err = (p - (s - bv)) + (c64 - bv)
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    up = np.nextafter(r, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r, np.float32(-np.inf)).astype(np.float64)
    lo = np.where(r64 <= s, r64, dn)
    hi = np.where(r64 >= s, r64, up)
    with np.errstate(invalid="ignore"):
        tie = (lo != hi) & (s - lo == hi - s)
    fix = tie & (err != 0)
    return np.where(fix, np.where(err > 0, hi, lo), r64).astype(np.float32)


def fused_sum_sq(e, w=None):
    """Squared errors of the last axis summed in order with one rounding per
    term: acc <- fma(t_i, e_i, acc), acc = 0 first, t_i = e_i (MSE) or
    fp32(w_i * e_i) (WMSE)."""
    e = np.asarray(e, dtype=np.float32)
    acc = np.zeros(e.shape[:-1], dtype=np.float32)
    for i in range(e.shape[-1]):
        ei = e[..., i]
        t = ei if w is None else (np.asarray(w, dtype=np.float32)[..., i] * ei).astype(np.float32)
        acc = fma_f32(t, ei, acc)
    return acc


def pack_nibbles(codes):
    """Two 4-bit codes per byte along the last axis: element 2k in the low
    nibble, element 2k+1 in the high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def _as_matrix_f32(x):
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("x must be a 2-D row-major matrix")
    if x.dtype != np.float32:
        x = x.astype(np.float32)          # bf16 inputs arrive already widened
    return x


def _first_argmin(losses, valid):
    """Index of the first valid candidate whose loss equals the minimum over
    the valid candidates (candidates along axis -1, in ascending order)."""
    masked = np.where(valid, losses, np.float32(np.inf))
    best = masked.min(axis=-1, keepdims=True)
    hit = valid & (masked == best)
    return np.argmax(hit, axis=-1)


@dataclass
class NVFP4Result:
    codes: np.ndarray        # uint8 [R, C/2], packed
    scales: np.ndarray       # uint8 [R, C/16], E4M3 patterns
    global_scale: np.float32
    block_loss: np.ndarray   # float32 [R, C/16]
    offsets: np.ndarray      # int8 [R, C/16], p* - base
    base: np.ndarray         # int64 [R, C/16], AbsMax pattern
    rotated: np.ndarray      # float32 [R, C], the values quantized


def sweep_blocks(ub, w, lo, hi):
    """Steps 3-6 of the NVFP4 sweep on blocks of magnitudes ub [..., 16] in
    units of S with per-element weights w (broadcastable, or None for MSE):
    returns the chosen pattern, its loss and the AbsMax base pattern."""
    a = ub.max(axis=-1)
    t = (a / np.float32(6.0)).astype(np.float32)
    base = np.maximum(F.e4m3_rne_pattern(t), 1)
    recip = F.e4m3_reciprocal_table()
    offsets = np.arange(lo, hi + 1)
    losses = np.empty(base.shape + (offsets.size,), dtype=np.float32)
    valid = np.empty(base.shape + (offsets.size,), dtype=bool)
    for k, o in enumerate(offsets):
        p = base + o
        ok = (p >= 1) & (p <= F.E4M3_MAX_PATTERN)
        pc = np.clip(p, 1, F.E4M3_MAX_PATTERN)
        V = F.E4M3_VALUES[pc][..., None]
        R = recip[pc][..., None]
        y = (ub * R).astype(np.float32)
        q = F.e2m1_value(F.e2m1_rne_index(y))
        d = (q * V).astype(np.float32)
        e = (ub - d).astype(np.float32)
        losses[..., k] = fused_sum_sq(e, None if w is None else np.broadcast_to(w, e.shape))
        valid[..., k] = ok
    k_best = _first_argmin(losses, valid)
    p_best = base + offsets[k_best]
    L_best = np.take_along_axis(losses, k_best[..., None], axis=-1)[..., 0]
    return p_best, L_best, base


def global_scale_nvfp4(x):
    """S = fp32(max|x| / 1536) for a float32 matrix ("Resumo Técnico:
    ScaleSweep", 2. Limites Teóricos, Escala Global)."""
    x = _as_matrix_f32(x)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    return np.float32(amax / np.float32(1536.0))


def quantize_nvfp4(x, importance=None, window=None, block=16,
                   global_scale=None, hadamard_n=0):
    """NVFP4 ScaleSweep of a float32 matrix (steps in the module doc).

    importance: per-column weights (length C) for WMSE, or None for MSE.
    window: (lo, hi) bit-pattern offsets; default (-3, 7) for MSE and
            (-8, 7) for WMSE.
    global_scale: use this S instead of computing it (float32 > 0).
    hadamard_n: rotate each row's n-groups first (0 = no rotation).
    """
    if block != 16:
        raise ValueError("NVFP4 blocks are 16 elements")
    x = _as_matrix_f32(x)
    if hadamard_n:
        x = block_hadamard(x, hadamard_n)
    rows, cols = x.shape
    if cols % block:
        raise ValueError("column count must be a multiple of the block size")
    wmse = importance is not None
    if window is None:
        window = (-8, 7) if wmse else (-3, 7)
    lo, hi = int(window[0]), int(window[1])
    if lo > 0 or hi < 0:
        raise ValueError("window must contain offset 0")

    if global_scale is None:
        S = global_scale_nvfp4(x)
    else:
        S = np.float32(global_scale)
    S_inv = np.float32(np.float32(1.0) / S) if S != 0 else np.float32(0.0)

    u = (np.abs(x) * S_inv).astype(np.float32)
    ub = u.reshape(rows, cols // block, block)
    w = np.asarray(importance, dtype=np.float32).reshape(cols // block, block) if wmse else None
    p_best, L_best, base = sweep_blocks(ub, w, lo, hi)
    recip = F.e4m3_reciprocal_table()
    R_best = recip[p_best][..., None]
    idx = F.e2m1_rne_index((ub * R_best).astype(np.float32))
    sign = np.signbit(x).reshape(rows, cols // block, block).astype(np.uint8)
    codes = (sign << 3) | idx
    SS = np.float32(S * S)
    return NVFP4Result(
        codes=pack_nibbles(codes.reshape(rows, cols)),
        scales=p_best.astype(np.uint8),
        global_scale=S,
        block_loss=(L_best * SS).astype(np.float32),
        offsets=(p_best - base).astype(np.int8),
        base=base,
        rotated=x,
    )


def dequantize_nvfp4(codes, scales, global_scale, block=16):
    """x_hat = (-1)**sign * fp32(fp32(q * V[p]) * S); q * V is exact."""
    c = unpack_nibbles(codes)
    rows, cols = c.shape
    sign = (c >> 3).astype(bool)
    q = F.e2m1_value(c & 7).reshape(rows, cols // block, block)
    V = F.E4M3_VALUES[np.asarray(scales, dtype=np.int64)][..., None]
    mag = ((q * V).astype(np.float32) * np.float32(global_scale)).astype(np.float32)
    mag = mag.reshape(rows, cols)
    return np.where(sign, -mag, mag).astype(np.float32)


@dataclass
class MXFP4Result:
    codes: np.ndarray        # uint8 [R, C/2]
    scales: np.ndarray       # uint8 [R, C/32], E8M0 bytes
    block_loss: np.ndarray   # float32 [R, C/32]
    offsets: np.ndarray      # int8 [R, C/32], E* - E_base
    e_base: np.ndarray       # int64 [R, C/32]
    rotated: np.ndarray


def mx_base_exponent(a):
    """E_base = min{E in Z : 6 * 2**E >= a}, clamped to [-127, 127]; found by
    searching E directly with exact float64 comparisons."""
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    safe = np.where(a > 0, a, 1.0)
    E = np.floor(np.log2(safe / 6.0)).astype(np.int64) - 1   # at or below the answer
    E = np.maximum(E, -200)
    while True:                     # raise E until 6 * 2**E >= a
        short = 6.0 * np.ldexp(1.0, E) < a
        if not short.any():
            break
        E = E + short
    while True:                     # lower E while 6 * 2**(E-1) still covers a
        slack = 6.0 * np.ldexp(1.0, E - 1) >= a
        slack &= a > 0
        if not slack.any():
            break
        E = E - slack
    E = np.where(a > 0, E, -127)
    return np.clip(E, -127, 127)


def sweep_blocks_mx(ub, w, lo, hi):
    """The MXFP4 exponent sweep on blocks of magnitudes ub [..., 32] with
    per-element weights w (broadcastable, or None for MSE): the base
    exponent, then for E = base + lo .. base + hi in ascending order the
    block's loss, the fused in-order sum over its 32 elements; returns
    (E*, its loss, the base exponent)."""
    E_base = mx_base_exponent(ub.max(axis=-1))
    offsets = np.arange(lo, hi + 1)
    losses = np.empty(E_base.shape + (offsets.size,), dtype=np.float32)
    valid = np.empty(E_base.shape + (offsets.size,), dtype=bool)
    for k, o in enumerate(offsets):
        E = E_base + o
        ok = (E >= -127) & (E <= 127)
        Ec = np.clip(E, -127, 127)
        down = F.pow2_f32(-Ec)[..., None]
        up = F.pow2_f32(Ec)[..., None]
        with np.errstate(over="ignore"):      # far below the base y overflows to inf: code 6
            y = (ub * down).astype(np.float32)
        q = F.e2m1_value(F.e2m1_rne_index(y))
        d = (q * up).astype(np.float32)
        e = (ub - d).astype(np.float32)
        losses[..., k] = fused_sum_sq(e, None if w is None else np.broadcast_to(w, e.shape))
        valid[..., k] = ok
    k_best = _first_argmin(losses, valid)
    E_best = E_base + offsets[k_best]
    L_best = np.take_along_axis(losses, k_best[..., None], axis=-1)[..., 0]
    return E_best, L_best, E_base


def quantize_mxfp4(x, importance=None, window=(-1, 0), block=32, hadamard_n=0):
    """MXFP4 exponent sweep of a float32 matrix (steps in the module doc)."""
    if block != 32:
        raise ValueError("MXFP4 blocks are 32 elements")
    x = _as_matrix_f32(x)
    if hadamard_n:
        x = block_hadamard(x, hadamard_n)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    rows, cols = x.shape
    if cols % block:
        raise ValueError("column count must be a multiple of the block size")
    lo, hi = int(window[0]), int(window[1])
    if lo > 0 or hi < 0:
        raise ValueError("window must contain offset 0")
    wmse = importance is not None
    if wmse:
        w = np.asarray(importance, dtype=np.float32).reshape(cols // block, block)

    u = np.abs(x).astype(np.float32)
    ub = u.reshape(rows, cols // block, block)
    E_best, L_best, E_base = sweep_blocks_mx(ub, w if wmse else None, lo, hi)
    y = (ub * F.pow2_f32(-E_best)[..., None]).astype(np.float32)
    idx = F.e2m1_rne_index(y)
    sign = np.signbit(x).reshape(rows, cols // block, block).astype(np.uint8)
    codes = (sign << 3) | idx
    return MXFP4Result(
        codes=pack_nibbles(codes.reshape(rows, cols)),
        scales=(E_best + 127).astype(np.uint8),
        block_loss=L_best.astype(np.float32),
        offsets=(E_best - E_base).astype(np.int8),
        e_base=E_base,
        rotated=x,
    )


def dequantize_mxfp4(codes, scales, block=32):
    """x_hat = (-1)**sign * q * 2**(b - 127) (exact)."""
    c = unpack_nibbles(codes)
    rows, cols = c.shape
    sign = (c >> 3).astype(bool)
    q = F.e2m1_value(c & 7).reshape(rows, cols // block, block)
    up = F.pow2_f32(np.asarray(scales, dtype=np.int64) - 127)[..., None]
    mag = (q * up).astype(np.float32).reshape(rows, cols)
    return np.where(sign, -mag, mag).astype(np.float32)

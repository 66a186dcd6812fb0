"""GPTQ with ScaleSweep group scales (oracle; test infrastructure).

"Resumo Técnico: ScaleSweep" (Principais Contribuições 2; Resultados,
Dados de Calibração): the bounded sweep chooses the NVFP4 block scales
inside GPTQ pipelines as well as RTN ones.  "Bridging the Gap ... Microscaling
FP4" (2. Metodologia, MR-GPTQ component 1): GPTQ's grid (group and global
scales) is chosen per format.  GPTQ itself is only named on the pages; it is
the published column-by-column quantization with error feedback through the
inverse Hessian, restated here:

  Given W (R x C), H = X^T X of calibration activations and U, the upper
  Cholesky factor of H^-1 (H^-1 = U^T U), columns are quantized in order.
  When column c opens a 16-column group, each row's E4M3 group scale is
  chosen by the sweep (oracle.quant.sweep_blocks) on the group's current,
  already error-corrected values; the global scale S is fixed from W before
  any update.  Column c is quantized at its group's scale, its scaled error
  err = fp32(fp32(W[:, c] - x_hat) * fp32(1 / U[c, c])) is recorded and
  every later column j of the same 128-column batch is updated with one
  fused multiply-add, W[:, j] <- fma(-err, U[c, j], W[:, j]); at the end of
  a batch the columns after it receive W <- fp32(W - Err @ U[batch, after])
  (the product taken in float64 here).
  Readings: S from the matrix before GPTQ; err uses the reciprocal of the
  diagonal; importance (WMSE) per column as given.

gptq_nvfp4_static / gptq_mxfp4_static add MR-GPTQ's static activation
reordering ("Bridging the Gap ... Microscaling FP4", 2. Metodologia,
component 2): the columns are processed in a given order while every group
keeps the scale chosen for it, before any update, in the stored order.
"""

import numpy as np

from . import formats as F
from .quant import (fma_f32, global_scale_nvfp4, pack_nibbles, sweep_blocks, sweep_blocks_mx, dequantize_nvfp4,
                    dequantize_mxfp4)

BATCH = 128


def gptq_nvfp4(W, U, importance=None, window=None, global_scale=None):
    """Returns (packed codes, scale patterns, S)."""
    W = np.array(W, dtype=np.float32, copy=True)
    U = np.asarray(U, dtype=np.float32)
    rows, cols = W.shape
    if cols % BATCH:
        raise ValueError("columns must be a multiple of 128")
    wmse = importance is not None
    lo, hi = window if window is not None else ((-8, 7) if wmse else (-3, 7))
    S = global_scale_nvfp4(W) if global_scale is None else np.float32(global_scale)
    S_inv = np.float32(np.float32(1.0) / S) if S != 0 else np.float32(0.0)
    recip = F.e4m3_reciprocal_table()
    rdiag = (np.float32(1.0) / np.diag(U)).astype(np.float32)
    imp = None if not wmse else np.asarray(importance, dtype=np.float32).reshape(cols // 16, 16)
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    for i1 in range(0, cols, BATCH):
        i2 = i1 + BATCH
        E = np.zeros((rows, BATCH), dtype=np.float32)
        for c in range(i1, i2):
            if c % 16 == 0:
                g = c // 16
                ub = (np.abs(W[:, c:c + 16]) * S_inv).astype(np.float32)[:, None, :]
                p, _, _ = sweep_blocks(ub, None if imp is None else imp[g][None, None, :], lo, hi)
                p = p[:, 0]
                scales[:, g] = p
                V = F.E4M3_VALUES[p]
                R = recip[p]
            w = W[:, c]
            u = (np.abs(w) * S_inv).astype(np.float32)
            idx = F.e2m1_rne_index((u * R).astype(np.float32))
            mag = ((F.e2m1_value(idx) * V).astype(np.float32) * S).astype(np.float32)
            what = np.where(np.signbit(w), -mag, mag).astype(np.float32)
            codes[:, c] = (np.signbit(w).astype(np.uint8) << 3) | idx
            err = ((w - what).astype(np.float32) * rdiag[c]).astype(np.float32)
            E[:, c - i1] = err
            if c + 1 < i2:
                W[:, c + 1:i2] = fma_f32(-err[:, None], U[c, c + 1:i2][None, :], W[:, c + 1:i2])
        if i2 < cols:
            acc = (E.astype(np.float64) @ U[i1:i2, i2:].astype(np.float64)).astype(np.float32)
            W[:, i2:] = (W[:, i2:] - acc).astype(np.float32)
    return pack_nibbles(codes), scales, S


def gptq_mxfp4(W, U, importance=None, window=(-1, 0)):
    """GPTQ with MXFP4 group scales ("Bridging the Gap ... Microscaling FP4",
    2. Metodologia, MR-GPTQ component 1: the grid is optimised per format,
    MXFP4 included).  The same column-by-column procedure as gptq_nvfp4 with
    MXFP4 groups: when column c opens a 32-column group, each row's E8M0
    exponent is the exponent sweep's choice (oracle.quant.sweep_blocks_mx) on
    the group's current values, from the base exponent over the window;
    x_hat = q * 2^E exactly (no global scale).  Returns (packed codes, E8M0
    scale bytes)."""
    W = np.array(W, dtype=np.float32, copy=True)
    U = np.asarray(U, dtype=np.float32)
    rows, cols = W.shape
    if cols % BATCH:
        raise ValueError("columns must be a multiple of 128")
    lo, hi = int(window[0]), int(window[1])
    wmse = importance is not None
    imp = None if not wmse else np.asarray(importance, dtype=np.float32).reshape(cols // 32, 32)
    rdiag = (np.float32(1.0) / np.diag(U)).astype(np.float32)
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    for i1 in range(0, cols, BATCH):
        i2 = i1 + BATCH
        E = np.zeros((rows, BATCH), dtype=np.float32)
        for c in range(i1, i2):
            if c % 32 == 0:
                g = c // 32
                ub = np.abs(W[:, c:c + 32]).astype(np.float32)[:, None, :]
                e_best = sweep_blocks_mx(ub, None if imp is None else imp[g][None, None, :], lo, hi)[0][:, 0]
                scales[:, g] = (e_best + 127).astype(np.uint8)
                down = F.pow2_f32(-e_best)
                up = F.pow2_f32(e_best)
            w = W[:, c]
            idx = F.e2m1_rne_index((np.abs(w) * down).astype(np.float32))
            mag = (F.e2m1_value(idx) * up).astype(np.float32)
            what = np.where(np.signbit(w), -mag, mag).astype(np.float32)
            codes[:, c] = (np.signbit(w).astype(np.uint8) << 3) | idx
            err = ((w - what).astype(np.float32) * rdiag[c]).astype(np.float32)
            E[:, c - i1] = err
            if c + 1 < i2:
                W[:, c + 1:i2] = fma_f32(-err[:, None], U[c, c + 1:i2][None, :], W[:, c + 1:i2])
        if i2 < cols:
            acc = (E.astype(np.float64) @ U[i1:i2, i2:].astype(np.float64)).astype(np.float32)
            W[:, i2:] = (W[:, i2:] - acc).astype(np.float32)
    return pack_nibbles(codes), scales


def _check_perm(perm, cols):
    perm = np.asarray(perm, dtype=np.int64).reshape(-1)
    if perm.size != cols or not np.array_equal(np.sort(perm), np.arange(cols)):
        raise ValueError("perm must be a permutation of the column indices")
    return perm


def _gptq_fixed_scales(Wp, U, xhat_of):
    """The column loop of gptq_nvfp4 on the columns of Wp in their given
    order, each rounded by xhat_of(c, w) -> (code, x_hat) at a scale fixed
    in advance; returns the codes in the order of Wp's columns."""
    Wp = np.array(Wp, dtype=np.float32, copy=True)
    rows, cols = Wp.shape
    rdiag = (np.float32(1.0) / np.diag(U)).astype(np.float32)
    codes = np.zeros((rows, cols), dtype=np.uint8)
    for i1 in range(0, cols, BATCH):
        i2 = i1 + BATCH
        E = np.zeros((rows, BATCH), dtype=np.float32)
        for c in range(i1, i2):
            w = Wp[:, c]
            codes[:, c], what = xhat_of(c, w)
            err = ((w - what).astype(np.float32) * rdiag[c]).astype(np.float32)
            E[:, c - i1] = err
            if c + 1 < i2:
                Wp[:, c + 1:i2] = fma_f32(-err[:, None], U[c, c + 1:i2][None, :], Wp[:, c + 1:i2])
        if i2 < cols:
            acc = (E.astype(np.float64) @ U[i1:i2, i2:].astype(np.float64)).astype(np.float32)
            Wp[:, i2:] = (Wp[:, i2:] - acc).astype(np.float32)
    return codes


def gptq_nvfp4_static(W, U, perm, importance=None, window=None, global_scale=None):
    """GPTQ with static activation reordering ("Bridging the Gap ...
    Microscaling FP4", 2. Metodologia, MR-GPTQ component 2: GPTQ's column
    reordering heuristic is applied once, when quantizing, so that inference
    shuffles nothing).  Reading: columns are processed in the order perm
    (GPTQ's heuristic puts the largest diagonal entries of H first; the
    caller computes perm and passes U, the upper Cholesky factor of the
    inverse of H permuted to that order), while the groups stay the
    contiguous 16-column blocks of the stored order.  Every group's scale is
    fixed before any update: the sweep (oracle.quant.sweep_blocks) on the
    weight as given, with S from that weight.  Column perm[j] is rounded at
    its stored group's scale when its turn j comes; errors and updates are
    those of gptq_nvfp4 in the processing order.  Returns (packed codes,
    scale patterns, S) in the stored order."""
    W0 = np.asarray(W, dtype=np.float32)
    U = np.asarray(U, dtype=np.float32)
    rows, cols = W0.shape
    if cols % BATCH:
        raise ValueError("columns must be a multiple of 128")
    perm = _check_perm(perm, cols)
    wmse = importance is not None
    lo, hi = window if window is not None else ((-8, 7) if wmse else (-3, 7))
    S = global_scale_nvfp4(W0) if global_scale is None else np.float32(global_scale)
    S_inv = np.float32(np.float32(1.0) / S) if S != 0 else np.float32(0.0)
    ub = (np.abs(W0) * S_inv).astype(np.float32).reshape(rows, cols // 16, 16)
    imp = None if not wmse else np.asarray(importance, dtype=np.float32).reshape(1, cols // 16, 16)
    scales = sweep_blocks(ub, imp, lo, hi)[0].astype(np.uint8)
    P = scales[:, perm // 16]                 # scale pattern of each processed column
    V_all = F.E4M3_VALUES[P]
    R_all = F.e4m3_reciprocal_table()[P]

    def xhat_of(c, w):
        u = (np.abs(w) * S_inv).astype(np.float32)
        idx = F.e2m1_rne_index((u * R_all[:, c]).astype(np.float32))
        mag = ((F.e2m1_value(idx) * V_all[:, c]).astype(np.float32) * S).astype(np.float32)
        code = (np.signbit(w).astype(np.uint8) << 3) | idx
        return code, np.where(np.signbit(w), -mag, mag).astype(np.float32)

    codes_p = _gptq_fixed_scales(W0[:, perm], U, xhat_of)
    codes = np.zeros_like(codes_p)
    codes[:, perm] = codes_p
    return pack_nibbles(codes), scales, S


def gptq_mxfp4_static(W, U, perm, importance=None, window=(-1, 0)):
    """gptq_nvfp4_static with MXFP4 groups (32 stored columns, E8M0
    exponents from oracle.quant.sweep_blocks_mx on the weight as given, no
    global scale): column perm[j] is rounded at 2^E of its stored group.
    Returns (packed codes, E8M0 bytes) in the stored order."""
    W0 = np.asarray(W, dtype=np.float32)
    U = np.asarray(U, dtype=np.float32)
    rows, cols = W0.shape
    if cols % BATCH:
        raise ValueError("columns must be a multiple of 128")
    perm = _check_perm(perm, cols)
    lo, hi = int(window[0]), int(window[1])
    imp = None if importance is None else np.asarray(importance, dtype=np.float32).reshape(1, cols // 32, 32)
    e_best = sweep_blocks_mx(np.abs(W0).reshape(rows, cols // 32, 32), imp, lo, hi)[0]
    scales = (e_best + 127).astype(np.uint8)
    Ecol = e_best[:, perm // 32]
    down_all, up_all = F.pow2_f32(-Ecol), F.pow2_f32(Ecol)

    def xhat_of(c, w):
        idx = F.e2m1_rne_index((np.abs(w) * down_all[:, c]).astype(np.float32))
        mag = (F.e2m1_value(idx) * up_all[:, c]).astype(np.float32)
        code = (np.signbit(w).astype(np.uint8) << 3) | idx
        return code, np.where(np.signbit(w), -mag, mag).astype(np.float32)

    codes_p = _gptq_fixed_scales(W0[:, perm], U, xhat_of)
    codes = np.zeros_like(codes_p)
    codes[:, perm] = codes_p
    return pack_nibbles(codes), scales


def proxy_loss(W0, codes, scales, S, H):
    """GPTQ's objective tr((W0 - W_hat) H (W0 - W_hat)^T) in float64 (NVFP4)."""
    D = np.asarray(W0, dtype=np.float64) - dequantize_nvfp4(codes, scales, S).astype(np.float64)
    return float(np.sum((D @ np.asarray(H, dtype=np.float64)) * D))


def proxy_loss_mx(W0, codes, scales, H):
    """The same objective for MXFP4 codes and E8M0 scales."""
    D = np.asarray(W0, dtype=np.float64) - dequantize_mxfp4(codes, scales).astype(np.float64)
    return float(np.sum((D @ np.asarray(H, dtype=np.float64)) * D))

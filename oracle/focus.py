"""FOCUS forward quantizer with coupled-relaxation coefficients (oracle; test
infrastructure).

"FOCUS: FP4 Optimization via Coupled-Relaxation and Dual-Granularity
Scaling", Metodologia 2 (Escalonamento de Relaxação Acoplada) and 3
(Escalonamento de Dupla Granularidade): the quantization scale of sub-block
k of a hardware block (16 for NVFP4, 32 for MXFP4; sub-blocks e.g. 8) is
S_q = S_dq * c_k, where S_dq is the block's stored, hardware-format
dequantization scale (E4M3 or E8M0) and c_k a full-precision FP16
coefficient; the codes are Q(W_k / (S_dq * c_k)) while dequantization keeps
using S_dq alone (4. Implantação e Compatibilidade: only FP4 codes and the
dequantization scales are deployed).

Reading, every float32 step rounded once (to nearest even):
  NVFP4: S_dq = V[p] * S (E4M3 block pattern p times the FP32 global scale);
         u = fp32(|x| * S_inv) as in the ScaleSweep path, S_inv = fp32(1/S)
         (0 if S = 0); Vc = fp32(V[p] * c_k); R = fp32(1 / Vc);
         y = fp32(u * R); q = RNE_E2M1(y).
  MXFP4: S_dq = 2**E (E8M0 byte E + 127); u = |x|; Vc = fp32(2**E * c_k);
         R = fp32(1 / Vc); y = fp32(u * R); q = RNE_E2M1(y).
  code = (signbit(x) << 3) | index(q).  With every c_k = 1 this is the
  round-to-nearest step of the scale search at the given scales.
  The dequantized output is the ordinary one: sign * fp32(fp32(q*V) * S)
  (NVFP4) or sign * q * 2**E (MXFP4).
Invalid data: a scale pattern outside 1..126 (NVFP4) or 255 (MXFP4), a
coefficient that is not finite and positive, or an infinite R.
"""

import numpy as np

from . import formats as F
from .quant import pack_nibbles, dequantize_mxfp4, dequantize_nvfp4


def quantize_given_scales(x, fmt, scales, global_scale=None, coeffs=None, sub=8):
    """Codes of x under per-sub-block quantization scales S_dq * c_k.

    x: float32 [R, C]; scales: uint8 [R, C/block]; coeffs: float16
    [R, C/sub] (None means every c_k = 1); returns (packed codes, dequantized
    float32 [R, C])."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    block = 16 if fmt == "nvfp4" else 32
    if cols % block or block % sub:
        raise ValueError("sub-blocks must tile the hardware blocks")
    scales = np.asarray(scales, dtype=np.int64)
    if coeffs is None:
        c = np.ones((rows, cols // sub), dtype=np.float32)
    else:
        c = np.asarray(coeffs, dtype=np.float16).astype(np.float32)
    if not np.all(np.isfinite(c) & (c > 0)):
        raise ValueError("coefficients must be finite and positive")
    per_sub = np.repeat(scales, block // sub, axis=1)          # block scale of each sub-block
    if fmt == "nvfp4":
        if np.any((scales < 1) | (scales > 126)):
            raise ValueError("E4M3 scale patterns must be 1..126")
        S = np.float32(global_scale)
        S_inv = np.float32(np.float32(1.0) / S) if S != 0 else np.float32(0.0)
        u = (np.abs(x) * S_inv).astype(np.float32)
        V = F.E4M3_VALUES[per_sub]
    elif fmt == "mxfp4":
        if np.any((scales < 0) | (scales > 254)):
            raise ValueError("E8M0 scale bytes must be 0..254")
        u = np.abs(x).astype(np.float32)
        V = F.pow2_f32(per_sub - 127)
    else:
        raise ValueError(fmt)
    Vc = (V * c).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        R = (np.float32(1.0) / Vc).astype(np.float32)
    if not np.all(np.isfinite(R)):
        raise ValueError("quantization scale too small: 1/(S_dq*c) overflows")
    R_el = np.repeat(R, sub, axis=1)
    y = (u * R_el).astype(np.float32)
    idx = F.e2m1_rne_index(y)
    codes = pack_nibbles((np.signbit(x).astype(np.uint8) << 3) | idx)
    if fmt == "nvfp4":
        xhat = dequantize_nvfp4(codes, scales.astype(np.uint8), np.float32(global_scale))
    else:
        xhat = dequantize_mxfp4(codes, scales.astype(np.uint8))
    return codes, xhat

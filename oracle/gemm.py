"""W4A4 matrix product of microscaled FP4 operands (oracle; test
infrastructure).

"Bridging the Gap Between Promise and Performance for Microscaling FP4
Quantization" (2. Metodologia; 3. QuTLASS): the quantized tensors are
consumed by a matrix product whose two operands are both FP4 (weights and
activations, W4A4).  A holds M activation rows and B holds N weight rows,
both over the same K input channels.  Each row is stored as E2M1 codes with
one scale per block of consecutive K elements (MXFP4: E8M0 per 32; NVFP4:
E4M3 per 16 times the tensor's FP32 global scale).  The product is
C = A_hat @ B_hat^T.  When a block rotation is used, both operands carry
the same block Hadamard along K, and it cancels in the product
(H H^T = I, same page, 2., micro-rotation).

What is computed here is that definition, written out:
  * every element is decoded exactly in float64:
      MXFP4  sign * q * 2**(b - 127), with b the E8M0 byte (255 is NaN);
      NVFP4  sign * q * E4M3(p) * S;
  * C = A_hat @ B_hat^T as one float64 matrix product (numpy).
Decoded elements have at most 2 (MXFP4) or 6 (NVFP4, without S)
significant bits, so every product is exact in float64.  The float64 sum
over K rounds far below the float32 accumulation of any GPU kernel, so for
testing this is the exact product.  ``abs_product`` gives
sum_k |a_ik| |b_jk|, the scale of the rounding-error bound.
"""

import numpy as np

from . import formats as F
from .quant import unpack_nibbles

E2M1_SIGNED64 = np.concatenate([F.E2M1_VALUES.astype(np.float64), -F.E2M1_VALUES.astype(np.float64)])
E4M3_WITH_NAN64 = np.concatenate([F.E4M3_VALUES64, [np.nan]])  # pattern 0x7F is NaN


def decode_mxfp4_64(codes, scales):
    """Exact float64 values of an MXFP4 tensor (rows x K)."""
    c = unpack_nibbles(np.asarray(codes, dtype=np.uint8))
    rows, k = c.shape
    b = np.asarray(scales, dtype=np.int64)
    if b.shape != (rows, k // 32):
        raise ValueError("scales must be rows x K/32")
    up = np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))
    return (E2M1_SIGNED64[c].reshape(rows, k // 32, 32) * up[..., None]).reshape(rows, k)


def decode_nvfp4_64(codes, scales, global_scale):
    """Exact float64 values of an NVFP4 tensor (rows x K)."""
    c = unpack_nibbles(np.asarray(codes, dtype=np.uint8))
    rows, k = c.shape
    p = np.asarray(scales, dtype=np.int64)
    if p.shape != (rows, k // 16):
        raise ValueError("scales must be rows x K/16")
    V = E4M3_WITH_NAN64[p & 0x7F] * np.where(p & 0x80, -1.0, 1.0)
    return (E2M1_SIGNED64[c].reshape(rows, k // 16, 16) * V[..., None]).reshape(rows, k) \
        * np.float64(np.float32(global_scale))


def gemm(a_hat, b_hat):
    """C = A_hat @ B_hat^T in float64."""
    return np.asarray(a_hat, dtype=np.float64) @ np.asarray(b_hat, dtype=np.float64).T


def abs_product(a_hat, b_hat):
    """sum_k |a_ik| |b_jk| in float64."""
    return np.abs(np.asarray(a_hat, dtype=np.float64)) @ np.abs(np.asarray(b_hat, dtype=np.float64)).T


def gemm_mxfp4(a_codes, a_scales, b_codes, b_scales):
    """C (M x N, float64) for MXFP4 operands A (M x K) and B (N x K)."""
    return gemm(decode_mxfp4_64(a_codes, a_scales), decode_mxfp4_64(b_codes, b_scales))


def gemm_nvfp4(a_codes, a_scales, a_global, b_codes, b_scales, b_global):
    """C (M x N, float64) for NVFP4 operands A (M x K) and B (N x K)."""
    return gemm(decode_nvfp4_64(a_codes, a_scales, a_global), decode_nvfp4_64(b_codes, b_scales, b_global))

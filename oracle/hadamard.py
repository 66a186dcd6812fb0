"""Block Hadamard rotation (oracle; test infrastructure).

"Bridging the Gap Between Promise and Performance for Microscaling FP4
Quantization", Resumo técnico, 2. Metodologia e Análise (MR-GPTQ component 3,
fused online rotations): weights and activations are rotated by block
Hadamard transforms ("micro-rotation") before FP4 quantization, which pulls
Laplace-like data towards a Normal shape.

Reading used here: each row of a row-major R x C matrix is split into
contiguous groups of n columns (n a power of two, 16 / 32 / 128 in the
workloads); each group is multiplied by the orthonormal Sylvester matrix
H_n / sqrt(n), in natural (Sylvester) order.  H_n is symmetric, so
x @ (H_n / sqrt(n)) equals the transform applied to each group as a column
vector, and the transform is its own inverse.

Two forms:
  * ``block_hadamard``       float32 fast transform with a fixed stage order:
                             stages h = 1, 2, 4, ..., n/2 replace (z_i, z_{i+h})
                             by (z_i + z_{i+h}, z_i - z_{i+h}) for every i with
                             i & h == 0, then every value is multiplied by
                             c_n = fp32(1/sqrt(n)).  This is the canonical
                             FP32 value the quantizer consumes.
  * ``block_hadamard_dense64`` float64 dense product with the Sylvester matrix,
                             the reference of record for tolerances.
"""

import numpy as np


def sylvester(n):
    """Sylvester Hadamard matrix H_n (entries +-1, int64), H_1 = [1],
    H_2k = [[H_k, H_k], [H_k, -H_k]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_scale_f32(n):
    """c_n = 1/sqrt(n) rounded once to float32 (computed in float64)."""
    return np.float32(1.0 / np.sqrt(np.float64(n)))


def block_hadamard(x, n):
    """Canonical float32 block Hadamard along the last axis (see module doc)."""
    z = np.array(x, dtype=np.float32, copy=True)
    cols = z.shape[-1]
    if n < 2 or n & (n - 1) or cols % n:
        raise ValueError("n must be a power of two >= 2 dividing the column count")
    g = z.reshape(z.shape[:-1] + (cols // n, n))
    h = 1
    while h < n:
        # view each group as (n / 2h) chunks of [first h | second h]
        v = g.reshape(g.shape[:-1] + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    z = g.reshape(z.shape) * hadamard_scale_f32(n)
    return z.astype(np.float32)


def block_hadamard_dense64(x, n):
    """float64 reference: each n-group times H_n / sqrt(n) (dense product)."""
    x = np.asarray(x, dtype=np.float64)
    cols = x.shape[-1]
    if cols % n:
        raise ValueError("n must divide the column count")
    hm = sylvester(n).astype(np.float64) / np.sqrt(np.float64(n))
    g = x.reshape(x.shape[:-1] + (cols // n, n))
    return (g @ hm).reshape(x.shape)

"""Seeded synthetic inputs for the FP4 quantizer (shared by tests and bench).

This module only draws random numbers and lays them out; it contains none of
the quantizer's arithmetic.  Both the CPU oracle and the HIP library receive
the tensors built here.

The shapes and distributions stand in for the LLM weights and activations
the pages quantize (their models and calibration sets are not used):
Gaussian initialisation, heavy-tailed Student-t weights, Laplace activations
with a few outlier channels ("Bridging the Gap ... Microscaling FP4",
2. Metodologia e Análise: native weights/activations modelled as Laplace with
outliers), and per-channel lognormal activation scales whose Gram diagonal
is the WMSE importance ("Resumo Técnico: ScaleSweep", 1. Objetivos de
Otimização).

Every generator is seeded with numpy PCG64 (``default_rng``) on the host,
except the 70B-shaped layer stream, which is drawn on the device with a
seeded ``torch.Generator`` per layer.  bf16 rounding uses torch's
round-to-nearest-even cast.
"""

import math

import numpy as np
import torch


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def gram_diag_importance(n_tokens, n_channels, seed):
    """imp_c = sum_t X[t, c]**2 for X = Z * lambda, Z ~ N(0, 1) of shape
    (n_tokens, n_channels), lambda_c = exp(N(0, 1)); float64, then float32."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n_tokens, n_channels))
    lam = np.exp(rng.standard_normal(n_channels))
    x = z * lam
    return np.einsum("tc,tc->c", x, x).astype(np.float32)


def rotated_gram_diag_importance(n_tokens, n_channels, n, seed):
    """Importance in the basis of an n-point block Hadamard rotation:
    imp_c = sum_t ((X @ blockdiag(H_n / sqrt(n)))[t, c])**2 with X drawn as in
    ``gram_diag_importance``.  The rotation of the calibration activations is
    a float64 dense product with scipy's Hadamard matrix."""
    import scipy.linalg

    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n_tokens, n_channels))
    lam = np.exp(rng.standard_normal(n_channels))
    x = (z * lam).reshape(n_tokens, n_channels // n, n)
    h = scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)
    xr = (x @ h).reshape(n_tokens, n_channels)
    return np.einsum("tc,tc->c", xr, xr).astype(np.float32)


# ------------------------------------------------------------- configs ----
def c1_weight():
    """256 x 1024 fp32, N(0, 0.02); 262 seeded entries (0.1%) times 20."""
    x = np.random.default_rng(101).standard_normal((256, 1024)) * 0.02
    pos = np.random.default_rng(102).choice(x.size, 262, replace=False)
    x.reshape(-1)[pos] *= 20.0
    return torch.from_numpy(x.astype(np.float32))


def c2_weight_and_importance():
    """4096 x 4096 bf16 Student-t (nu = 4) scaled to std 0.02 (t4 has variance
    2, so the factor is 0.02 / sqrt(2)); importance from 512 x 4096
    lognormal-scaled Gaussian activations."""
    w = np.random.default_rng(201).standard_t(4, (4096, 4096)) * (0.02 / math.sqrt(2.0))
    rng_z = np.random.default_rng(202)
    rng_l = np.random.default_rng(203)
    z = rng_z.standard_normal((512, 4096))
    lam = np.exp(rng_l.standard_normal(4096))
    x = z * lam
    imp = np.einsum("tc,tc->c", x, x).astype(np.float32)
    return _bf16(w), torch.from_numpy(imp)


def c3_activation():
    """8192 tokens x 4096 channels bf16, Laplace(0, 1), 8 seeded outlier
    channels times 50."""
    x = np.random.default_rng(301).laplace(0.0, 1.0, (8192, 4096))
    ch = np.random.default_rng(302).choice(4096, 8, replace=False)
    x[:, ch] *= 50.0
    return _bf16(x)


LAYER_8B = {  # name: (rows = output dim, cols = input dim)
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336),
}
_SEEDS_8B = {"q": 401, "k": 402, "v": 403, "o": 404, "gate": 405, "up": 406, "down": 407}
# importance groups: matrices that read the same input share one vector
_IMP_8B = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gateup", "up": "gateup", "down": "down"}
_IMP_SEEDS_8B = {"qkv": 411, "gateup": 412, "o": 413, "down": 414}


def c4_matrix(name):
    """One 8B-shaped decoder matrix, bf16 N(0, 0.02)."""
    rows, cols = LAYER_8B[name]
    w = np.random.default_rng(_SEEDS_8B[name]).standard_normal((rows, cols)) * 0.02
    return _bf16(w)


def c4_importance(name):
    """Importance for a c4 matrix: 2048 tokens of lognormal-scaled Gaussian
    activations of the matrix's input width."""
    group = _IMP_8B[name]
    cols = LAYER_8B[name][1]
    return torch.from_numpy(gram_diag_importance(2048, cols, _IMP_SEEDS_8B[group]))


LAYER_70B = {
    "q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
    "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672),
}
_IMP_70B = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gateup", "up": "gateup", "down": "down"}
_IMP_SEEDS_70B = {"qkv": 591, "o": 592, "gateup": 593, "down": 594}
C5_LAYERS = 80
C5_HADAMARD = 16


def c5_importance(name):
    """Rotated-basis importance (16-point block Hadamard) for a 70B matrix."""
    group = _IMP_70B[name]
    cols = LAYER_70B[name][1]
    return torch.from_numpy(rotated_gram_diag_importance(2048, cols, C5_HADAMARD, _IMP_SEEDS_70B[group]))


def c5_matrix(layer, name, device, shape=None):
    """One 70B-shaped matrix of layer ``layer``, drawn on ``device``:
    N(0, 0.02) with a Bernoulli(5e-4) mask of entries times 30, bf16.
    ``shape`` overrides the 70B shape (small streams in tests)."""
    order = list(LAYER_70B)
    g = torch.Generator(device=device)
    g.manual_seed(500000 + 1000 * layer + order.index(name))
    rows, cols = shape if shape is not None else LAYER_70B[name]
    w = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32) * 0.02
    mask = torch.rand((rows, cols), generator=g, device=device) < 5e-4
    w = torch.where(mask, w * 30.0, w)
    return w.to(torch.bfloat16)


# ----------------------------------------------------- W4A4 layer ----
W4A4_TOKENS = 8192
# activation inputs of an 8B-shaped decoder layer and the matrices that read them
W4A4_INPUTS = {"attn_in": 4096, "attn_out": 4096, "mlp_in": 4096, "mlp_mid": 14336}
W4A4_READS = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "attn_out",
              "gate": "mlp_in", "up": "mlp_in", "down": "mlp_mid"}


def w4a4_activation(name, device, tokens=W4A4_TOKENS):
    """Activations of one layer input, drawn on ``device``: Laplace(0, 1) as
    the difference of two Exp(1) draws, -log(1 - r) with r a seeded uniform
    in [0, 1) (always finite), 8 seeded outlier channels times 50 (the c3
    recipe at the input's width), bf16."""
    cols = W4A4_INPUTS[name]
    g = torch.Generator(device=device)
    g.manual_seed(700 + list(W4A4_INPUTS).index(name))
    r1 = torch.rand((tokens, cols), generator=g, device=device, dtype=torch.float32)
    r2 = torch.rand((tokens, cols), generator=g, device=device, dtype=torch.float32)
    x = torch.log1p(-r2) - torch.log1p(-r1)
    ch = torch.randperm(cols, generator=g, device=device)[:8]
    x[:, ch] *= 50.0
    return x.to(torch.bfloat16)


# ------------------------------------------------------- small cases ----
def random_matrix(rows, cols, seed, dist="normal", scale=0.02, dtype=torch.float32):
    """Generic seeded test matrix (normal, t4, laplace)."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((rows, cols))
    elif dist == "t4":
        x = rng.standard_t(4, (rows, cols)) / math.sqrt(2.0)
    elif dist == "laplace":
        x = rng.laplace(0.0, 1.0, (rows, cols))
    else:
        raise ValueError(dist)
    x = (x * scale).astype(np.float32)
    t = torch.from_numpy(x)
    return t.to(dtype) if dtype != torch.float32 else t


def random_importance(cols, seed, zero_frac=0.0):
    """Lognormal-squared per-column weights, some set to zero."""
    rng = np.random.default_rng(seed)
    w = np.exp(2.0 * rng.standard_normal(cols)).astype(np.float32)
    if zero_frac:
        w[rng.random(cols) < zero_frac] = 0.0
    return torch.from_numpy(w)


# ------------------------------------------------------------ GPTQ ----
def calibration_activations(n_tokens, n_channels, seed, corr=0.5):
    """Correlated synthetic calibration activations: lognormal channel
    scales times Gaussian tokens mixed by a random low-rank factor."""
    rng = np.random.default_rng(seed)
    lam = np.exp(rng.standard_normal(n_channels))
    rank = max(1, n_channels // 16)
    z = rng.standard_normal((n_tokens, n_channels)) * (1 - corr) \
        + rng.standard_normal((n_tokens, rank)) @ rng.standard_normal((rank, n_channels)) * (corr / np.sqrt(rank))
    return z * lam


def act_order_and_factor(x, damp=0.01):
    """GPTQ's processing order for static reordering and the factor that goes
    with it: perm lists the columns by descending diagonal of H = X^T X (ties
    by index), and U is the upper Cholesky factor of (Hp + damp * mean(diag
    H) * I)^-1 for Hp = H[perm][:, perm], as float32.  Returns (H, perm as
    int32, U).  numpy's sort and dense linear algebra (input preparation,
    not the path)."""
    x = np.asarray(x, dtype=np.float64)
    H = x.T @ x
    perm = np.argsort(-np.diag(H), kind="stable").astype(np.int32)
    Hp = H[perm][:, perm]
    Hd = Hp + damp * np.mean(np.diag(H)) * np.eye(H.shape[0])
    L = np.linalg.cholesky(Hd)
    Linv = np.linalg.inv(L)
    U = np.linalg.cholesky(Linv.T @ Linv).T
    return H, perm, np.ascontiguousarray(U, dtype=np.float32)


def hessian_and_factor(x, damp=0.01):
    """H = X^T X (float64) and U, the upper Cholesky factor of (H + damp *
    mean(diag H) * I)^-1, as float32: the inputs GPTQ consumes.  Computed
    with numpy's dense linear algebra (input preparation, not the path)."""
    x = np.asarray(x, dtype=np.float64)
    H = x.T @ x
    Hd = H + damp * np.mean(np.diag(H)) * np.eye(H.shape[0])
    L = np.linalg.cholesky(Hd)
    Linv = np.linalg.inv(L)
    Hinv = Linv.T @ Linv
    U = np.linalg.cholesky(Hinv).T
    return H, np.ascontiguousarray(U, dtype=np.float32)

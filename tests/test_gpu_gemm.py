"""GPU parity of the W4A4 MXFP4 matrix product (fp4q_gemm_mxfp4) against the
float64 oracle (oracle/gemm.py) on the same seeded operands.

Bar:
  * bit-exact whenever every partial sum is exactly representable in float32.
    With all scales 2^0, every product is a multiple of 1/4 of magnitude
    <= 36, so any sum of up to 4096 of them is exact in float32, whatever
    the order.  This case checks the operand, scale and accumulator layouts
    element by element.
  * otherwise |C - C_exact| <= (2 ceil(K/64) + 2) * 2^-24 * sum_k |a_ik b_jk|.
    That is one float32 rounding for each 64-element step's sum, one for
    adding it to the accumulator, and one each for alpha and the store.
  * bfloat16 output: additionally the bfloat16 unit roundoff of |C| (8-bit
    significand: 2^-8 relative).
Operands are random E2M1 bytes with scales around 2^0, the oracle's MXFP4
quantization of Laplace activations with outlier channels and Gaussian
weights (block Hadamard 32 on both), and, at full size in the bench's launch
configuration, random operands compared on sampled rows.
"""

import math

import numpy as np
import pytest
import torch

from oracle import gemm as GM
from oracle import quant as Q

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fq():
    import fp4_post_quantization_amd as fq
    return fq


def _fq_lib():
    from fp4_post_quantization_amd import _lib
    return _lib.load()


def _rand_mx(rng, rows, k, lo=120, hi=134):
    codes = rng.integers(0, 256, (rows, k // 2)).astype(np.uint8)
    scales = rng.integers(lo, hi + 1, (rows, k // 32)).astype(np.uint8)
    return codes, scales


def _dev(*arrs):
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrs)


def _bound(a_hat, b_hat, k):
    return (2 * math.ceil(k / 64) + 2) * 2.0 ** -24 * GM.abs_product(a_hat, b_hat)


def _run(ac, as_, bc, bs, out_dtype=torch.float32, alpha=1.0):
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    c = _fq().gemm_mxfp4((a, asd), (b, bsd), alpha=alpha, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


def _check(c, ac, as_, bc, bs, k, bf16=False, rows=None):
    A = GM.decode_mxfp4_64(ac, as_)
    B = GM.decode_mxfp4_64(bc, bs)
    if rows is not None:
        A = A[rows]
    ref = GM.gemm(A, B)
    tol = _bound(A, B, k)
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    err = np.abs(c - ref)
    bad = err > tol
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outside the bound; worst ratio "
                           f"{np.max(err / np.maximum(tol, 1e-300)):.3g}")
    return float(np.max(err / np.maximum(tol, 1e-300)))


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (5, 7, 64), (33, 65, 128), (64, 64, 256), (130, 257, 160),
                                   (257, 129, 4096), (300, 260, 1056), (96, 640, 2048)])
def test_gemm_exact_when_partial_sums_are_representable(m, n, k):
    rng = np.random.default_rng(1000 + m + n + k)
    ac, _ = _rand_mx(rng, m, k)
    bc, _ = _rand_mx(rng, n, k)
    as_ = np.full((m, k // 32), 127, np.uint8)
    bs = np.full((n, k // 32), 127, np.uint8)
    c = _run(ac, as_, bc, bs)
    ref = GM.gemm_mxfp4(ac, as_, bc, bs)
    np.testing.assert_array_equal(c, ref)


@pytest.mark.parametrize("m,n,k", [(5, 7, 64), (33, 65, 128), (130, 257, 160), (257, 129, 4096),
                                   (300, 260, 1056), (512, 1024, 512)])
def test_gemm_random_scales_within_bound(m, n, k):
    rng = np.random.default_rng(2000 + m + n + k)
    ac, as_ = _rand_mx(rng, m, k, 100, 150)
    bc, bs = _rand_mx(rng, n, k, 100, 150)
    _check(_run(ac, as_, bc, bs), ac, as_, bc, bs, k)


def test_gemm_bf16_output_and_alpha():
    rng = np.random.default_rng(3001)
    m, n, k = 200, 300, 512
    ac, as_ = _rand_mx(rng, m, k)
    bc, bs = _rand_mx(rng, n, k)
    c = _run(ac, as_, bc, bs, out_dtype=torch.bfloat16)
    _check(c, ac, as_, bc, bs, k, bf16=True)
    # alpha = 0.5 only halves, exactly
    c1 = _run(ac, as_, bc, bs)
    c2 = _run(ac, as_, bc, bs, alpha=0.5)
    np.testing.assert_array_equal(c2, 0.5 * c1)


def test_gemm_leading_dimension_and_untouched_padding():
    fq = _fq()
    rng = np.random.default_rng(3002)
    m, n, k = 70, 90, 256
    ac, as_ = _rand_mx(rng, m, k)
    bc, bs = _rand_mx(rng, n, k)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    big = torch.full((m, 128), 7.0, device=DEV)
    fq.gemm_mxfp4((a, asd), (b, bsd), out=big[:, :n])
    torch.cuda.synchronize()
    out = big.cpu().numpy()
    assert np.all(out[:, n:] == 7.0)
    _check(out[:, :n].astype(np.float64), ac, as_, bc, bs, k)


def test_gemm_nan_scale_byte():
    """E8M0 byte 255 encodes NaN; every output that reads it is NaN."""
    rng = np.random.default_rng(3003)
    m, n, k = 40, 50, 128
    ac, as_ = _rand_mx(rng, m, k)
    bc, bs = _rand_mx(rng, n, k)
    as_[3, 2] = 255
    c = _run(ac, as_, bc, bs)
    ref = GM.gemm_mxfp4(ac, as_, bc, bs)
    assert np.all(np.isnan(c[3])) and np.all(np.isnan(ref[3]))
    mask = np.ones(m, bool)
    mask[3] = False
    assert np.all(np.isfinite(c[mask]))


def test_gemm_of_quantized_rotated_operands():
    """W4A4 on the oracle's MXFP4 quantization of rotated activations and
    weights: the GPU product matches the oracle's product of the same codes,
    and both approximate X W^T (the rotation cancels)."""
    x = np.random.default_rng(3004).laplace(0, 1, (192, 1024)).astype(np.float32)
    x[:, [5, 300, 777]] *= 50
    w = (np.random.default_rng(3005).standard_normal((320, 1024)) * 0.02).astype(np.float32)
    qa = Q.quantize_mxfp4(x, window=(0, 0), hadamard_n=32)
    qb = Q.quantize_mxfp4(w, window=(-1, 0), hadamard_n=32)
    c = _run(qa.codes, qa.scales, qb.codes, qb.scales)
    _check(c, qa.codes, qa.scales, qb.codes, qb.scales, 1024)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(c - ref) / np.linalg.norm(ref) < 0.2


@pytest.mark.parametrize("m,n,k", [(64, 96, 256), (300, 260, 1024), (1024, 640, 512), (4096, 4096, 768)])
def test_gemm_scale_reorganisation_is_transparent(m, n, k):
    """Stage-major scales (workspace given) and row-major scales (none) give
    identical products for every tile configuration."""
    rng = np.random.default_rng(3008 + m + k)
    ac, as_ = _rand_mx(rng, m, k, 90, 160)
    bc, bs = _rand_mx(rng, n, k, 90, 160)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    fq = _fq()
    c1 = fq.gemm_mxfp4((a, asd), (b, bsd), use_workspace=True)
    c2 = fq.gemm_mxfp4((a, asd), (b, bsd), use_workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    rows = np.arange(0, m, max(1, m // 40))
    _check(c1[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64), ac, as_, bc, bs, k, rows=rows)


# up to 64 tokens: the few-token kernel (16 or 32 columns per workgroup, K split over its waves, up to
# four 16-row tiles)
@pytest.mark.parametrize("m,n,k", [(1, 16, 512), (3, 100, 4096), (16, 4096, 4096), (7, 1000, 14336),
                                   (16, 33, 8192), (1, 4096, 1536), (5, 8200, 1024), (16, 14336, 4096),
                                   (2, 8192, 14336), (17, 1000, 4096), (33, 300, 4096), (64, 4096, 4096),
                                   (48, 2000, 8192), (40, 4000, 512)])
def test_gemm_few_tokens_exact(m, n, k):
    rng = np.random.default_rng(3400 + m + n + k)
    ac, _ = _rand_mx(rng, m, k)
    bc, _ = _rand_mx(rng, n, k)
    as_ = np.full((m, k // 32), 127, np.uint8)
    bs = np.full((n, k // 32), 127, np.uint8)
    np.testing.assert_array_equal(_run(ac, as_, bc, bs), GM.gemm_mxfp4(ac, as_, bc, bs))


@pytest.mark.parametrize("m,n,k,out_dtype", [(1, 4096, 14336, torch.float32), (5, 300, 4096, torch.bfloat16),
                                             (16, 2048, 2048, torch.float32), (9, 8232, 2048, torch.bfloat16),
                                             (20, 4096, 14336, torch.float32), (33, 1024, 8192, torch.bfloat16)])
def test_gemm_few_tokens_within_bound(m, n, k, out_dtype):
    fq = _fq()
    rng = np.random.default_rng(3500 + m + n + k)
    ac, as_ = _rand_mx(rng, m, k, 100, 150)
    bc, bs = _rand_mx(rng, n, k, 100, 150)
    A = GM.decode_mxfp4_64(ac, as_)
    B = GM.decode_mxfp4_64(bc, bs)
    ref = -1.5 * GM.gemm(A, B)
    tol = 1.5 * _bound(A, B, k)
    if out_dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    big = torch.full((m, n + 8), 7.0, device=DEV, dtype=out_dtype)
    fq.gemm_mxfp4((a, asd), (b, bsd), alpha=-1.5, out_dtype=out_dtype, out=big[:, :n])
    torch.cuda.synchronize()
    got = big.float().cpu().numpy().astype(np.float64)
    assert (np.abs(got[:, :n] - ref) <= tol).all()
    assert (got[:, n:] == 7.0).all()  # the padding past n is untouched


# few-token products the few-token kernel does not take (K not a multiple of 512, or more row-tile
# steps than it holds): K split over workgroups (the workspace holds the partial sums)
@pytest.mark.parametrize("m,n,k", [(40, 700, 14336), (5, 1000, 4352), (64, 2048, 14336), (50, 4096, 12800)])
def test_gemm_few_tokens_split_k_exact(m, n, k):
    rng = np.random.default_rng(3100 + m + n + k)
    ac, _ = _rand_mx(rng, m, k)
    bc, _ = _rand_mx(rng, n, k)
    as_ = np.full((m, k // 32), 127, np.uint8)
    bs = np.full((n, k // 32), 127, np.uint8)
    np.testing.assert_array_equal(_run(ac, as_, bc, bs), GM.gemm_mxfp4(ac, as_, bc, bs))


@pytest.mark.parametrize("m,n,k,out_dtype", [(40, 2000, 14336, torch.bfloat16), (17, 1024, 5376, torch.float32),
                                             (64, 512, 14336, torch.float32), (1, 4096, 14592, torch.float32)])
def test_gemm_few_tokens_split_k_within_bound(m, n, k, out_dtype):
    fq = _fq()
    rng = np.random.default_rng(3200 + m + n + k)
    ac, as_ = _rand_mx(rng, m, k, 100, 150)
    bc, bs = _rand_mx(rng, n, k, 100, 150)
    lib = __import__("fp4_post_quantization_amd._lib", fromlist=["load"]).load()
    # the workspace for these shapes holds split partial sums
    assert lib.fp4q_gemm_mxfp4_workspace_bytes(m, n, k) >= 2 * m * n * 4
    c = _run(ac, as_, bc, bs, out_dtype=out_dtype, alpha=0.75)
    A = GM.decode_mxfp4_64(ac, as_)
    B = GM.decode_mxfp4_64(bc, bs)
    ref = 0.75 * GM.gemm(A, B)
    tol = 0.75 * _bound(A, B, k)
    if out_dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    assert (np.abs(c - ref) <= tol).all()
    # without a workspace: one accumulation over all of K, also within the bound
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    c2 = fq.gemm_mxfp4((a, asd), (b, bsd), alpha=0.75, out_dtype=out_dtype, use_workspace=False)
    assert (np.abs(c2.float().cpu().numpy().astype(np.float64) - ref) <= tol).all()


def test_gemm_output_beyond_2gib_sampled_rows():
    """C of 32800 x 16384 float32 (2.15 GB): rows past the 2^31-byte offset are
    written where they belong.  Unit scales make every sum exact, so the
    sampled rows are compared bit for bit with the oracle."""
    fq = _fq()
    m, n, k = 32800, 16384, 256
    g = torch.Generator(device=DEV)
    g.manual_seed(3300)
    a = torch.randint(0, 256, (m, k // 2), dtype=torch.uint8, device=DEV, generator=g)
    b = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=DEV, generator=g)
    sa = torch.full((m, k // 32), 127, dtype=torch.uint8, device=DEV)
    sb = torch.full((n, k // 32), 127, dtype=torch.uint8, device=DEV)
    c = fq.gemm_mxfp4((a, sa), (b, sb))
    torch.cuda.synchronize()
    pick = np.array([0, 32767, 32768, 32769, 32799])
    ref = GM.gemm_mxfp4(a.cpu().numpy()[pick], sa.cpu().numpy()[pick], b.cpu().numpy(), sb.cpu().numpy())
    got = c[torch.from_numpy(pick).to(DEV)].cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got, ref)


def test_gemm_large_tiles_with_k_tail():
    """K not a multiple of 128 with enough rows and columns for 256 x 256
    tiles: the register-staged path with its zero-filled K tail; sampled rows
    against the oracle, bit-exact with unit scales."""
    rng = np.random.default_rng(3007)
    m, n, k = 4096, 4096, 1056
    ac, _ = _rand_mx(rng, m, k)
    bc, _ = _rand_mx(rng, n, k)
    as_ = np.full((m, k // 32), 127, np.uint8)
    bs = np.full((n, k // 32), 127, np.uint8)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    c_all = _fq().gemm_mxfp4((a, asd), (b, bsd))
    torch.cuda.synchronize()
    rows = np.sort(np.concatenate([[0, 255, 256, 4095], rng.choice(m, 28, replace=False)]))
    c = c_all[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    ref = GM.gemm(GM.decode_mxfp4_64(ac, as_)[rows], GM.decode_mxfp4_64(bc, bs))
    np.testing.assert_array_equal(c, ref)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gemm_full_size_sampled_rows(out_dtype):
    """8192 tokens x 14336 outputs x 4096 inputs (an 8B-shaped up/gate
    projection) in the bench's launch configuration; 48 sampled rows are
    checked against the oracle."""
    rng = np.random.default_rng(3006)
    m, n, k = 8192, 14336, 4096
    ac, as_ = _rand_mx(rng, m, k)
    bc, bs = _rand_mx(rng, n, k)
    c_all = torch.empty((m, n), dtype=out_dtype, device=DEV)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    _fq().gemm_mxfp4((a, asd), (b, bsd), out=c_all)
    torch.cuda.synchronize()
    rows = np.sort(np.concatenate([[0, 1, 255, 256, 4095, 8191], rng.choice(m, 42, replace=False)]))
    c = c_all[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    _check(c, ac, as_, bc, bs, k, bf16=out_dtype == torch.bfloat16, rows=rows)


# More tiles than the CUs hold at once: each workgroup walks several tiles, fetching the next
# tile's first stage while it finishes the current one and staging the output through a ring slot.
# Ragged edges in both dimensions, one stage per tile (K = 256) and several, stage-major and
# row-major scales; 256 x 256 tiles (289 and 306 of them, one workgroup per CU) and 128 x 128 tiles
# (528, two workgroups per CU).
@pytest.mark.parametrize("m,n,k,use_ws", [(4100, 4200, 256, True), (4100, 4200, 256, False),
                                          (4352, 4160, 768, True), (4352, 4160, 768, False),
                                          (4100, 2000, 256, False), (4100, 2000, 768, True)])
def test_gemm_persistent_tiles_exact(m, n, k, use_ws):
    rng = np.random.default_rng(3100 + m + k + use_ws)
    ac, _ = _rand_mx(rng, m, k)
    bc, _ = _rand_mx(rng, n, k)
    as_ = np.full((m, k // 32), 127, np.uint8)
    bs = np.full((n, k // 32), 127, np.uint8)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    fq = _fq()
    c32 = fq.gemm_mxfp4((a, asd), (b, bsd), use_workspace=use_ws)
    c16 = fq.gemm_mxfp4((a, asd), (b, bsd), use_workspace=use_ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.sort(np.unique(np.concatenate([[0, 255, 256, 4095, 4096, m - 1], rng.choice(m, 40, replace=False)])))
    ref = GM.gemm(GM.decode_mxfp4_64(ac, as_)[rows], GM.decode_mxfp4_64(bc, bs))
    r = torch.from_numpy(rows).to(DEV)
    np.testing.assert_array_equal(c32[r].cpu().numpy().astype(np.float64), ref)
    # exact float32 sums, so the bfloat16 output is their round-to-nearest-even
    ref16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(c16[r].cpu(), ref16)


# ----------------------------------------------------------- NVFP4 operands ----
# Bar: the operands are decoded exactly (q * E4M3 in bfloat16) and each product is exact in the
# float32 accumulator, so |C - C_exact| <= (2 ceil(K/16) + 3) * 2^-24 * sum_k |a_ik b_jk|, with
# one rounding for each 16-element step's sum and one for adding it, plus fp32(S_a S_b), the final
# multiply and the store; bit-exact when every partial sum is representable (unit block and global
# scales).


def _rand_nv(rng, rows, k, lo=40, hi=80):
    codes = rng.integers(0, 256, (rows, k // 2)).astype(np.uint8)
    scales = rng.integers(lo, hi + 1, (rows, k // 16)).astype(np.uint8)
    return codes, scales


def _run_nv(ac, as_, ag, bc, bs, bg, out_dtype=torch.float32):
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    c = _fq().gemm_nvfp4((a, asd, float(ag)), (b, bsd, float(bg)), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


def _check_nv(c, ac, as_, ag, bc, bs, bg, k, bf16=False, rows=None):
    A = GM.decode_nvfp4_64(ac, as_, ag)
    B = GM.decode_nvfp4_64(bc, bs, bg)
    if rows is not None:
        A = A[rows]
    ref = GM.gemm(A, B)
    tol = (2 * math.ceil(k / 16) + 3) * 2.0 ** -24 * GM.abs_product(A, B)
    if bf16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    err = np.abs(c - ref)
    bad = err > tol
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outside the bound; worst ratio "
                           f"{np.max(err / np.maximum(tol, 1e-300)):.3g}")


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (5, 7, 48), (33, 65, 128), (130, 257, 176), (257, 129, 2048),
                                   (300, 260, 1040)])
def test_gemm_nvfp4_exact_with_unit_scales(m, n, k):
    rng = np.random.default_rng(4000 + m + n + k)
    ac, _ = _rand_nv(rng, m, k)
    bc, _ = _rand_nv(rng, n, k)
    as_ = np.full((m, k // 16), 0x38, np.uint8)  # E4M3 1.0
    bs = np.full((n, k // 16), 0x38, np.uint8)
    c = _run_nv(ac, as_, 1.0, bc, bs, 1.0)
    np.testing.assert_array_equal(c, GM.gemm_nvfp4(ac, as_, np.float32(1), bc, bs, np.float32(1)))


@pytest.mark.parametrize("m,n,k", [(5, 7, 48), (130, 257, 176), (257, 129, 2048), (512, 1024, 512)])
def test_gemm_nvfp4_random_scales_within_bound(m, n, k):
    rng = np.random.default_rng(5000 + m + n + k)
    ac, as_ = _rand_nv(rng, m, k, 1, 126)
    bc, bs = _rand_nv(rng, n, k, 1, 126)
    ag, bg = np.float32(0.0137), np.float32(0.71)
    _check_nv(_run_nv(ac, as_, ag, bc, bs, bg), ac, as_, ag, bc, bs, bg, k)


def test_gemm_nvfp4_of_quantized_operands_and_nan_scale():
    """The oracle's NVFP4 sweep of t4 weights and Laplace activations: the GPU
    product matches the oracle's product of the same codes and tracks X W^T;
    an E4M3 NaN scale byte gives a NaN row."""
    rng = np.random.default_rng(5100)
    x = rng.laplace(0, 1, (96, 512)).astype(np.float32)
    w = (rng.standard_t(4, (160, 512)) * 0.02).astype(np.float32)
    qa, qb = Q.quantize_nvfp4(x), Q.quantize_nvfp4(w)
    c = _run_nv(qa.codes, qa.scales, qa.global_scale, qb.codes, qb.scales, qb.global_scale)
    _check_nv(c, qa.codes, qa.scales, qa.global_scale, qb.codes, qb.scales, qb.global_scale, 512)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(c - ref) / np.linalg.norm(ref) < 0.2
    sc = qa.scales.copy()
    sc[7, 3] = 0x7F
    c2 = _run_nv(qa.codes, sc, qa.global_scale, qb.codes, qb.scales, qb.global_scale)
    assert np.all(np.isnan(c2[7]))
    mask = np.ones(96, bool)
    mask[7] = False
    assert np.all(np.isfinite(c2[mask]))


# at most 32 tokens (64 on outputs of at most 4096 columns) with K a multiple of 256: the few-token
# kernel (codes decoded to float16 in registers, float16 matrix cores, no workspace)
@pytest.mark.parametrize("m,n,k", [(1, 16, 256), (3, 100, 4096), (16, 4096, 4096), (7, 1000, 14336),
                                   (16, 33, 8192), (2, 8200, 1024), (16, 14336, 4096), (9, 512, 16384),
                                   (17, 1000, 4096), (33, 300, 2048), (64, 4096, 4096), (20, 2000, 8192),
                                   (32, 8200, 4096), (20, 4096, 14336), (60, 2048, 14336), (5, 512, 32768)])
def test_gemm_nvfp4_few_tokens_exact(m, n, k):
    """The last three split K over two or four workgroups per column tile (partial sums in the
    workspace, added in K order)."""
    rng = np.random.default_rng(5300 + m + n + k)
    ac, _ = _rand_nv(rng, m, k)
    bc, _ = _rand_nv(rng, n, k)
    as_ = np.full((m, k // 16), 0x38, np.uint8)  # E4M3 1.0
    bs = np.full((n, k // 16), 0x38, np.uint8)
    assert _fq_lib().fp4q_gemm_nvfp4_workspace_bytes(m, n, k) < (m + n) * k * 2
    c = _run_nv(ac, as_, 1.0, bc, bs, 1.0)
    np.testing.assert_array_equal(c, GM.gemm_nvfp4(ac, as_, np.float32(1), bc, bs, np.float32(1)))


def _rand_nv_any_scale(rng, rows, k):
    """Codes and scale bytes over every non-NaN E4M3 pattern: zero, subnormal, normal, both signs."""
    codes = rng.integers(0, 256, (rows, k // 2)).astype(np.uint8)
    scales = rng.integers(0, 256, (rows, k // 16)).astype(np.uint8)
    scales[(scales & 0x7F) == 0x7F] = 0xB8  # -1.0 in place of NaN
    return codes, scales


@pytest.mark.parametrize("m,n,k,out_dtype", [(1, 4096, 14336, torch.float32), (5, 300, 4096, torch.bfloat16),
                                             (16, 2048, 2048, torch.float32), (9, 8232, 2048, torch.bfloat16),
                                             (48, 3000, 2048, torch.bfloat16), (24, 4096, 14336, torch.bfloat16)])
def test_gemm_nvfp4_few_tokens_within_bound(m, n, k, out_dtype):
    rng = np.random.default_rng(5400 + m + n + k)
    ac, as_ = _rand_nv_any_scale(rng, m, k)
    bc, bs = _rand_nv_any_scale(rng, n, k)
    ag, bg = np.float32(0.0137), np.float32(-0.71)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    big = torch.full((m, n + 8), 7.0, device=DEV, dtype=out_dtype)
    _fq().gemm_nvfp4((a, asd, float(ag)), (b, bsd, float(bg)), out=big[:, :n])
    torch.cuda.synchronize()
    got = big.float().cpu().numpy().astype(np.float64)
    _check_nv(got[:, :n], ac, as_, ag, bc, bs, bg, k, bf16=out_dtype == torch.bfloat16)
    assert (got[:, n:] == 7.0).all()  # the padding past n is untouched


def test_gemm_nvfp4_few_tokens_nan_scales():
    """An E4M3 NaN scale byte (0x7F or 0xFF) in A gives a NaN row, in B a NaN column."""
    rng = np.random.default_rng(5500)
    m, n, k = 6, 96, 1024
    ac, as_ = _rand_nv(rng, m, k)
    bc, bs = _rand_nv(rng, n, k)
    as_[2, 5] = 0x7F
    bs[40, 63] = 0xFF
    c = _run_nv(ac, as_, 0.5, bc, bs, 2.0)
    assert np.all(np.isnan(c[2])) and np.all(np.isnan(c[:, 40]))
    keep = np.ones((m, n), bool)
    keep[2] = False
    keep[:, 40] = False
    assert np.all(np.isfinite(c[keep]))
    _check_nv(c[keep].reshape(m - 1, n - 1), ac[[0, 1, 3, 4, 5]], as_[[0, 1, 3, 4, 5]], 0.5,
              np.delete(bc, 40, 0), np.delete(bs, 40, 0), 2.0, k)


# K a multiple of 128 (and 16-byte aligned codes), products below 256 x 256 tiles on every CU: codes
# staged in LDS, decoded in registers, float16 matrix cores (128 x 128 and 64 x 64 tiles); one
# product of the large-tile size checks the decode pass that takes those
@pytest.mark.parametrize("m,n,k", [(4096, 4096, 256), (1536, 1408, 384), (200, 300, 640), (33, 65, 128)])
def test_gemm_nvfp4_ring_exact(m, n, k):
    rng = np.random.default_rng(5600 + m + n + k)
    ac, _ = _rand_nv(rng, m, k)
    bc, _ = _rand_nv(rng, n, k)
    as_ = np.full((m, k // 16), 0x38, np.uint8)
    bs = np.full((n, k // 16), 0x38, np.uint8)
    c = _run_nv(ac, as_, 1.0, bc, bs, 1.0)
    np.testing.assert_array_equal(c, GM.gemm_nvfp4(ac, as_, np.float32(1), bc, bs, np.float32(1)))


@pytest.mark.parametrize("m,n,k,out_dtype", [(4096, 4096, 256, torch.bfloat16), (1536, 1408, 384, torch.float32),
                                             (200, 300, 640, torch.bfloat16)])
def test_gemm_nvfp4_ring_within_bound(m, n, k, out_dtype):
    rng = np.random.default_rng(5700 + m + n + k)
    ac, as_ = _rand_nv_any_scale(rng, m, k)
    bc, bs = _rand_nv_any_scale(rng, n, k)
    ag, bg = np.float32(0.0213), np.float32(-1.37)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    big = torch.full((m, n + 8), 7.0, device=DEV, dtype=out_dtype)
    _fq().gemm_nvfp4((a, asd, float(ag)), (b, bsd, float(bg)), out=big[:, :n])
    torch.cuda.synchronize()
    got = big.float().cpu().numpy().astype(np.float64)
    _check_nv(got[:, :n], ac, as_, ag, bc, bs, bg, k, bf16=out_dtype == torch.bfloat16)
    assert (got[:, n:] == 7.0).all()  # the padding past n is untouched


def test_gemm_nvfp4_persistent_tiles_exact():
    """bfloat16 output over more 256 x 256 tiles than CUs (the decode pass and the bf16 ring walking
    several tiles per workgroup), ragged in both dimensions, unit scales: every sum is exact, so the
    output is its round-to-nearest-even."""
    rng = np.random.default_rng(5650)
    m, n, k = 4100, 4200, 512
    ac, _ = _rand_nv(rng, m, k)
    bc, _ = _rand_nv(rng, n, k)
    as_ = np.full((m, k // 16), 0x38, np.uint8)
    bs = np.full((n, k // 16), 0x38, np.uint8)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    c16 = _fq().gemm_nvfp4((a, asd, 1.0), (b, bsd, 1.0), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.sort(np.unique(np.concatenate([[0, 255, 256, 4095, 4096, m - 1], rng.choice(m, 40, replace=False)])))
    ref = GM.gemm(GM.decode_nvfp4_64(ac, as_, np.float32(1))[rows], GM.decode_nvfp4_64(bc, bs, np.float32(1)))
    ref16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(c16[torch.from_numpy(rows).to(DEV)].cpu(), ref16)


def test_gemm_nvfp4_full_size_sampled_rows():
    """8192 x 14336 x 4096 with bf16 output in the launch configuration of
    the large-tile path; 40 sampled rows against the oracle."""
    rng = np.random.default_rng(5200)
    m, n, k = 8192, 14336, 4096
    ac, as_ = _rand_nv(rng, m, k)
    bc, bs = _rand_nv(rng, n, k)
    ag, bg = np.float32(0.003), np.float32(0.02)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    c_all = _fq().gemm_nvfp4((a, asd, float(ag)), (b, bsd, float(bg)), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.sort(np.concatenate([[0, 255, 256, 8191], rng.choice(m, 36, replace=False)]))
    c = c_all[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    _check_nv(c, ac, as_, ag, bc, bs, bg, k, bf16=True, rows=rows)


def test_single_row_output_view_with_any_row_stride():
    """A one-row output view whose row stride is below N (a transposed
    column) is written like a dense row: its row stride is never used."""
    rng = np.random.default_rng(77)
    k, n = 1024, 96
    ac, as_ = _rand_mx(rng, 1, k)
    bc, bs = _rand_mx(rng, n, k)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    fq = _fq()
    ref = fq.gemm_mxfp4((a, asd), (b, bsd))
    out = torch.empty((n, 1), device=DEV).t()
    assert out.shape == (1, n) and out.stride(0) < n
    got = fq.gemm_mxfp4((a, asd), (b, bsd), out=out)
    nac, nas = _rand_nv(rng, 1, k)
    nbc, nbs = _rand_nv(rng, n, k)
    na, nasd, nb, nbsd = _dev(nac, nas, nbc, nbs)
    nref = fq.gemm_nvfp4((na, nasd, 1.0), (nb, nbsd, 1.0))
    nout = torch.empty((n, 1), device=DEV).t()
    ngot = fq.gemm_nvfp4((na, nasd, 1.0), (nb, nbsd, 1.0), out=nout)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr() and torch.equal(got, ref)
    assert ngot.data_ptr() == nout.data_ptr() and torch.equal(ngot, nref)
    with pytest.raises(ValueError):
        fq.gemm_mxfp4((a.expand(3, -1), asd.expand(3, -1)), (b, bsd), out=torch.empty(n, device=DEV).expand(3, n))


def test_operands_on_another_device_are_refused():
    rng = np.random.default_rng(78)
    ac, as_ = _rand_mx(rng, 4, 512)
    bc, bs = _rand_mx(rng, 64, 512)
    a, asd, b, bsd = _dev(ac, as_, bc, bs)
    fq = _fq()
    with pytest.raises(ValueError):
        fq.gemm_mxfp4((a, asd), (b.cpu(), bsd))
    with pytest.raises(ValueError):
        fq.gemm_mxfp4((a, asd), (b, bsd), out=torch.empty((4, 64)))
    with pytest.raises(ValueError):
        fq.gemm_mxfp4((a.cpu(), asd.cpu()), (b.cpu(), bsd.cpu()))
    nac, nas = _rand_nv(rng, 4, 512)
    nbc, nbs = _rand_nv(rng, 64, 512)
    na, nasd, nb, nbsd = _dev(nac, nas, nbc, nbs)
    with pytest.raises(ValueError):
        fq.gemm_nvfp4((na, nasd, 1.0), (nb, nbsd.cpu(), 1.0))
    x = torch.randn(8, 64, device=DEV)
    with pytest.raises(ValueError):
        fq.quantize_nvfp4(x, ws=torch.zeros(fq._lib.load().fp4q_workspace_bytes(), dtype=torch.uint8))
    torch.cuda.synchronize()

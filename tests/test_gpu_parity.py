"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Bar: codes, scales, offsets, the global scale and per-block losses are
bit-exact on unrotated inputs.  With a block Hadamard rotation the rotated
values must be within 1e-5 of the float64 dense product (per block,
relative to the block's largest magnitude), at most 1e-4 of the codes may
differ and per-block losses must agree within 1e-5 relative; the GPU rotation
is additionally checked to reproduce the oracle's float32 fast transform bit
for bit, in which case everything downstream is bit-exact too.
"""

import json

import numpy as np
import pytest
import torch

import workloads as W
from oracle import focus as FO
from oracle import gptq as GQ
from oracle import formats as F
from oracle import quant as Q
from oracle import hadamard as OH

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fp4():
    import fp4_post_quantization_amd as fq
    return fq


def _np(t):
    return t.detach().cpu().numpy()


def _host_f32(x):
    return x.detach().float().cpu().numpy()


def _assert_equal(name, got, ref):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.dtype.kind == "f":
        same = (got.view(np.uint32) == ref.astype(np.float32).view(np.uint32))
    else:
        same = got == ref
    if not np.all(same):
        idx = np.argwhere(~same)
        i = tuple(idx[0])
        raise AssertionError(f"{name}: {idx.shape[0]} of {same.size} differ; first at {i}: "
                             f"gpu={got[i]!r} oracle={ref[i]!r}")


def _check_nvfp4(res, ref, rows=None):
    sl = slice(None) if rows is None else rows
    _assert_equal("global_scale", np.float32(_np(res.global_scale)[0]), np.float32(ref.global_scale))
    _assert_equal("codes", _np(res.codes)[sl], ref.codes)
    _assert_equal("scales", _np(res.scales)[sl], ref.scales)
    _assert_equal("offsets", _np(res.offsets)[sl], ref.offsets)
    _assert_equal("block_loss", _np(res.block_loss)[sl], ref.block_loss)


def _check_mxfp4(res, ref, rows=None):
    sl = slice(None) if rows is None else rows
    _assert_equal("codes", _np(res.codes)[sl], ref.codes)
    _assert_equal("scales", _np(res.scales)[sl], ref.scales)
    _assert_equal("offsets", _np(res.offsets)[sl], ref.offsets)
    _assert_equal("block_loss", _np(res.block_loss)[sl], ref.block_loss)


def _run_nvfp4(x, imp=None, window=None, had=0, gs=None):
    fq = _fp4()
    xd = x.to(DEV)
    impd = None if imp is None else imp.to(DEV)
    res = fq.quantize_nvfp4(xd, impd, window=window, hadamard_n=had, global_scale=gs, check=True)
    torch.cuda.synchronize()
    return res


def _oracle_nvfp4(x, imp=None, window=None, had=0, gs=None):
    return Q.quantize_nvfp4(_host_f32(x), None if imp is None else imp.numpy(), window=window,
                            hadamard_n=had, global_scale=gs)


# ------------------------------------------------------- small shapes ----
SHAPES = [(1, 16), (3, 32), (3, 48), (257, 4112), (64, 1024), (5, 2048)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("wmse", [False, True])
def test_nvfp4_small_shapes(rows, cols, dtype, wmse):
    x = W.random_matrix(rows, cols, seed=rows * 7919 + cols, dist="t4", dtype=dtype)
    imp = W.random_importance(cols, seed=cols, zero_frac=0.05) if wmse else None
    _check_nvfp4(_run_nvfp4(x, imp), _oracle_nvfp4(x, imp))


@pytest.mark.parametrize("window", [(0, 0), (-3, 7), (-8, 7), (-1, 2), (-126, 126)])
def test_nvfp4_windows(window):
    x = W.random_matrix(96, 512, seed=31, dist="laplace")
    x[5, 17] = 3.0  # a tensor-maximum block whose window clips at 0x7E
    imp = W.random_importance(512, seed=32)
    for im in (None, imp):
        _check_nvfp4(_run_nvfp4(x, im, window=window), _oracle_nvfp4(x, im, window=window))


def test_nvfp4_leading_dimension_larger_than_cols():
    big = W.random_matrix(33, 1056, seed=41, dtype=torch.bfloat16)
    fq = _fp4()
    xd = big.to(DEV)[:, :1024]                  # ld = 1056 > cols = 1024
    res = fq.quantize_nvfp4(xd, check=True)
    ref = _oracle_nvfp4(big[:, :1024].contiguous())
    _check_nvfp4(res, ref)


@pytest.mark.parametrize("had", [16, 128])
def test_nvfp4_rotated_leading_dimension_larger_than_cols(had):
    big = W.random_matrix(37, 1280, seed=43, dist="laplace", dtype=torch.bfloat16)
    imp = W.random_importance(1024, seed=44)
    fq = _fp4()
    res = fq.quantize_nvfp4(big.to(DEV)[:, :1024], imp.to(DEV), hadamard_n=had, check=True)
    torch.cuda.synchronize()
    _check_nvfp4(res, _oracle_nvfp4(big[:, :1024].contiguous(), imp, had=had))


def test_nvfp4_given_scale():
    x = W.random_matrix(40, 256, seed=42)
    S = np.float32(0.37 / 1536)
    _check_nvfp4(_run_nvfp4(x, gs=float(S)), _oracle_nvfp4(x, gs=S))


# -------------------------------------------------------- edge tensors ----
def test_edge_zero_tensor_and_negative_zero():
    x = torch.zeros(4, 64)
    x[1, 3] = -0.0
    res = _run_nvfp4(x)
    _check_nvfp4(res, _oracle_nvfp4(x))
    assert float(_np(res.global_scale)[0]) == 0.0


def test_edge_single_nonzero():
    x = torch.zeros(3, 48)
    x[2, 40] = -1e-3
    _check_nvfp4(_run_nvfp4(x), _oracle_nvfp4(x))
    m = torch.zeros(3, 64)
    m[0, 5] = 7.0
    fq = _fp4()
    r = fq.quantize_mxfp4(m.to(DEV), check=True)
    _check_mxfp4(r, Q.quantize_mxfp4(m.numpy()))


def test_edge_exact_ties():
    """With S = 1 and a power-of-two base scale, u * R hits every E2M1
    midpoint exactly: ties must go to the even code on both sides."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows = []
    for scale in (1.0, 0.5, 2.0 ** -7, 4.0):
        r = np.zeros(16, dtype=np.float32)
        r[0] = 6 * scale
        r[1:8] = np.float32(mids) * scale
        r[8:15] = -np.float32(mids) * scale
        r[15] = np.float32(2.9) * scale
        rows.append(r)
    x = torch.from_numpy(np.stack(rows))
    _check_nvfp4(_run_nvfp4(x, gs=1.0), _oracle_nvfp4(x, gs=np.float32(1.0)))
    _check_nvfp4(_run_nvfp4(x, window=(0, 0), gs=1.0), _oracle_nvfp4(x, window=(0, 0), gs=np.float32(1.0)))
    xm = torch.from_numpy(np.concatenate([np.stack(rows), np.stack(rows)], axis=1))
    fq = _fp4()
    r = fq.quantize_mxfp4(xm.to(DEV), window=(0, 0), check=True)
    _check_mxfp4(r, Q.quantize_mxfp4(xm.numpy(), window=(0, 0)))


# rows near the float32 maximum overflow S*S and the losses in the oracle on purpose (both sides
# must then agree on inf / NaN), so numpy's overflow warnings are expected here
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_edge_subnormal_bases_and_bf16_extremes():
    rng = np.random.default_rng(51)
    x = (rng.standard_normal((16, 256)) * 1e-7).astype(np.float32)
    x[0, 0] = 1.0                                  # most blocks get subnormal E4M3 bases
    x[1, :16] = np.float32(3.0e38)                 # near the bf16 / fp32 maximum
    x[2, :32] = np.float32(1e-39)                  # float32 subnormals
    xt = torch.from_numpy(x)
    _check_nvfp4(_run_nvfp4(xt), _oracle_nvfp4(xt))
    xb = xt.to(torch.bfloat16)
    _check_nvfp4(_run_nvfp4(xb), _oracle_nvfp4(xb))
    fq = _fp4()
    r = fq.quantize_mxfp4(xb.to(DEV), check=True)
    _check_mxfp4(r, Q.quantize_mxfp4(_host_f32(xb)))


def test_edge_zero_importance_columns():
    x = W.random_matrix(20, 256, seed=52)
    imp = W.random_importance(256, seed=53)
    imp[:64] = 0.0
    _check_nvfp4(_run_nvfp4(x, imp), _oracle_nvfp4(x, imp))


def test_empty_rows():
    fq = _fp4()
    x = torch.empty(0, 64, device=DEV)
    r = fq.quantize_nvfp4(x, check=True)
    torch.cuda.synchronize()
    assert r.codes.shape == (0, 32)
    assert float(r.global_scale.item()) == 0.0


# ------------------------------------------------------- data errors ----
def test_data_errors_set_status():
    fq = _fp4()
    x = W.random_matrix(8, 64, seed=54).to(DEV)
    x[3, 7] = float("nan")
    with pytest.raises(fq.FP4QError, match="non-finite"):
        fq.quantize_nvfp4(x, check=True)
    with pytest.raises(fq.FP4QError, match="non-finite"):
        fq.quantize_mxfp4(x, check=True)
    y = W.random_matrix(8, 64, seed=55).to(DEV)
    imp = torch.ones(64, device=DEV)
    imp[9] = -1.0
    with pytest.raises(fq.FP4QError, match="importance"):
        fq.quantize_nvfp4(y, imp, check=True)
    with pytest.raises(fq.FP4QError, match="global scale"):
        fq.quantize_nvfp4(y, global_scale=float("inf"), check=True)
    # a clean call afterwards resets the status word
    fq.quantize_nvfp4(y, check=True)


# ------------------------------------ the global scale alone, two streams ----
@pytest.mark.parametrize("dtype,had,ld_extra", [(torch.bfloat16, 0, 0), (torch.float32, 0, 32),
                                                (torch.bfloat16, 16, 0), (torch.float32, 128, 64)])
def test_global_scale_alone_matches_oracle(dtype, had, ld_extra):
    x = W.random_matrix(67, 1024 + ld_extra, seed=80 + had, dist="laplace", dtype=dtype)
    fq = _fp4()
    S = fq.global_scale_nvfp4(x.to(DEV)[:, :1024], had)
    torch.cuda.synchronize()
    ref = np.float32(_oracle_nvfp4(x[:, :1024].contiguous(), had=had).global_scale)
    assert _np(S).view(np.uint32)[0] == np.array([ref]).view(np.uint32)[0], (float(_np(S)[0]), float(ref))


def test_global_scale_of_empty_tensor_is_zero():
    fq = _fp4()
    S = torch.full((1,), 5.0, device=DEV)
    fq.global_scale_nvfp4(torch.zeros((0, 64), device=DEV), out=S)
    torch.cuda.synchronize()
    assert float(S[0]) == 0.0


def test_given_scale_from_the_scale_pass_is_one_call():
    """The global scale alone, then the sweep with that scale given: every
    output field identical to one quantize_nvfp4 call computing S."""
    fq = _fp4()
    specs = [(64, 1024, "t4", torch.bfloat16), (300, 512, "laplace", torch.float32), (1, 2048, "normal", torch.bfloat16)]
    for i, (r, c, d, dt) in enumerate(specs):
        x = W.random_matrix(r, c, seed=95 + i, dist=d, dtype=dt).to(DEV)
        for had, imp in ((0, W.random_importance(c, seed=99 + i).to(DEV)), (16, None)):
            S = fq.global_scale_nvfp4(x, had)
            two = fq.quantize_nvfp4(x, imp, hadamard_n=had, global_scale=S)
            one = fq.quantize_nvfp4(x, imp, hadamard_n=had)
            torch.cuda.synchronize()
            for f in ("codes", "scales", "global_scale", "block_loss", "offsets"):
                assert torch.equal(getattr(two, f), getattr(one, f)), (i, had, f)


def test_deterministic():
    fq = _fp4()
    x = W.random_matrix(512, 2048, seed=56, dtype=torch.bfloat16).to(DEV)
    imp = W.random_importance(2048, seed=57).to(DEV)
    a = fq.quantize_nvfp4(x, imp)
    b = fq.quantize_nvfp4(x, imp)
    torch.cuda.synchronize()
    for f in ("codes", "scales", "offsets", "block_loss", "global_scale"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_broadcast_and_strided_views_are_read_as_their_values():
    """A row-broadcast view (row stride 0) and a column-strided view reach
    the library as dense copies, so it never reads past the storage."""
    fq = _fp4()
    row = W.random_matrix(1, 512, seed=60, dtype=torch.bfloat16).to(DEV)
    view = row.expand(37, 512)
    dense = view.contiguous()
    a = fq.quantize_nvfp4(view, check=True)
    b = fq.quantize_nvfp4(dense, check=True)
    wide = W.random_matrix(20, 1024, seed=61).to(DEV)
    c = fq.quantize_mxfp4(wide[:, ::2], check=True)
    d = fq.quantize_mxfp4(wide[:, ::2].contiguous(), check=True)
    torch.cuda.synchronize()
    for f in ("codes", "scales", "offsets", "block_loss", "global_scale"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    for f in ("codes", "scales", "offsets", "block_loss"):
        assert torch.equal(getattr(c, f), getattr(d, f)), f
    _check_nvfp4(a, _oracle_nvfp4(dense.cpu()))


def test_caller_buffers_are_checked_before_the_library_writes():
    fq = _fp4()
    x = W.random_matrix(32, 256, seed=62).to(DEV)
    good = fq.quantize_nvfp4(x)
    bad = [good._replace(codes=good.codes[:, :64]),
           good._replace(scales=good.scales.to(torch.int8)),
           good._replace(block_loss=torch.empty((32, 32), device=DEV)[:, ::2]),
           good._replace(offsets=good.offsets.cpu())]
    for out in bad:
        with pytest.raises(ValueError):
            fq.quantize_nvfp4(x, out=out)
    mx = fq.quantize_mxfp4(x)
    with pytest.raises(ValueError):
        fq.quantize_mxfp4(x, out=mx._replace(scales=good.scales))
    with pytest.raises(ValueError):
        fq.dequantize("nvfp4", good.codes, good.scales[:, :8], good.global_scale)
    with pytest.raises(ValueError):
        fq.block_hadamard(x, 16, out=torch.empty((32, 128), device=DEV))
    with pytest.raises(ValueError):
        fq.global_scale_nvfp4(x, out=torch.empty(1, dtype=torch.float64, device=DEV))
    with pytest.raises(ValueError):
        fq.quantize_relaxed(x, good.scales, global_scale=good.global_scale, out_codes=good.codes[:16])
    torch.cuda.synchronize()


def test_binding_passes_the_current_stream():
    fq = _fp4()
    d = torch.device(DEV)
    assert fq._stream(d) == int(torch.cuda.current_stream(d).cuda_stream)
    side = torch.cuda.Stream(d)
    with torch.cuda.stream(side):
        assert fq._stream(d) == int(side.cuda_stream) == int(torch.cuda.current_stream(d).cuda_stream)
    assert fq._stream(d) != int(side.cuda_stream)


def test_default_workspace_is_per_stream():
    """Calls that pass no workspace on two streams use two workspaces (the
    global-max partials and status word of one cannot be overwritten by the
    other), and both give the default stream's result."""
    fq = _fp4()
    x = W.random_matrix(300, 1024, seed=58, dtype=torch.bfloat16).to(DEV)
    imp = W.random_importance(1024, seed=59).to(DEV)
    main = fq.workspace(DEV)
    assert fq.workspace(DEV) is main
    ref = fq.quantize_nvfp4(x, imp, check=True)
    side = [torch.cuda.Stream(DEV) for _ in range(2)]
    torch.cuda.synchronize()
    outs = []
    for s in side:
        with torch.cuda.stream(s):
            assert fq.workspace(DEV) is not main
            outs.append(fq.quantize_nvfp4(x, imp))
    torch.cuda.synchronize()
    assert fq.workspace(DEV) is main
    with torch.cuda.stream(side[0]):
        ws0 = fq.workspace(DEV)
    with torch.cuda.stream(side[1]):
        assert fq.workspace(DEV) is not ws0
    for o in outs:
        for f in ("codes", "scales", "offsets", "block_loss", "global_scale"):
            assert torch.equal(getattr(o, f), getattr(ref, f)), f


# ------------------------------------------------------------- MXFP4 ----
@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (257, 4128), (64, 1024)])
@pytest.mark.parametrize("window", [(-1, 0), (0, 0), (-3, 2)])
def test_mxfp4_small(rows, cols, window):
    x = W.random_matrix(rows, cols, seed=rows + cols, dist="laplace", scale=1.0, dtype=torch.bfloat16)
    fq = _fp4()
    r = fq.quantize_mxfp4(x.to(DEV), window=window, check=True)
    _check_mxfp4(r, Q.quantize_mxfp4(_host_f32(x), window=window))
    imp = W.random_importance(cols, seed=cols + 1)
    r = fq.quantize_mxfp4(x.to(DEV), imp.to(DEV), window=window, check=True)
    _check_mxfp4(r, Q.quantize_mxfp4(_host_f32(x), imp.numpy(), window=window))


def test_e2m1_rounding_dense_through_mxfp4():
    """The E2M1 rounding of the library on every float32 within 2**14 steps
    of each midpoint and on every 256th float32 in [0, 6]: MXFP4 blocks led
    by 6.0 get the scale 2**0 under the AbsMax window, so each code is the
    E2M1 rounding of |x| itself.  Signs alternate to cover the sign bit."""
    mids = F.E2M1_MIDPOINTS.view(np.uint32).astype(np.int64)
    near = (mids[:, None] + np.arange(-2**14, 2**14)[None, :]).ravel()
    sweep = np.arange(0, int(np.float32(6.0).view(np.uint32)) + 1, 256, dtype=np.int64)
    vals = np.concatenate([near, sweep]).astype(np.uint32).view(np.float32)
    vals = vals[(vals >= 0) & (vals <= 6)]
    n = -(-vals.size // 31)
    body = np.zeros(n * 31, dtype=np.float32)
    body[:vals.size] = vals
    body[1::2] *= -1
    x = np.empty((n, 32), dtype=np.float32)
    x[:, 0] = 6.0
    x[:, 1:] = body.reshape(n, 31)
    fq = _fp4()
    r = fq.quantize_mxfp4(torch.from_numpy(x).to(DEV), window=(0, 0), check=True)
    torch.cuda.synchronize()
    ref = Q.quantize_mxfp4(x, window=(0, 0))
    assert np.all(ref.scales == 127)
    _check_mxfp4(r, ref)


# ---------------------------------------------------------- dequant ----
def test_dequantize_matches_oracle():
    fq = _fp4()
    x = W.random_matrix(77, 512, seed=61, dist="t4")
    r = fq.quantize_nvfp4(x.to(DEV))
    out = fq.dequantize("nvfp4", r.codes, r.scales, r.global_scale)
    ref = Q.dequantize_nvfp4(_np(r.codes), _np(r.scales), _np(r.global_scale)[0])
    _assert_equal("nvfp4 dequant", _np(out), ref)
    m = fq.quantize_mxfp4(x.to(DEV))
    out = fq.dequantize("mxfp4", m.codes, m.scales)
    _assert_equal("mxfp4 dequant", _np(out), Q.dequantize_mxfp4(_np(m.codes), _np(m.scales)))


# ---------------------------------------------------------- Hadamard ----
@pytest.mark.parametrize("n", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_hadamard(n, dtype):
    fq = _fp4()
    x = W.random_matrix(131, 1024, seed=n, dist="laplace", scale=1.0, dtype=dtype)
    z = _np(fq.block_hadamard(x.to(DEV), n))
    xf = _host_f32(x)
    _assert_equal("fwht", z, OH.block_hadamard(xf, n))
    ref = OH.block_hadamard_dense64(xf, n)
    blk = np.abs(ref).reshape(131, -1, n).max(-1, keepdims=True)
    err = np.abs(z - ref).reshape(131, -1, n)
    assert np.all(err <= 1e-5 * blk)


def _rotated_checks(res, ref_fn, x_host, n, imp=None):
    """Spec tolerances for rotated inputs, then bit-exactness."""
    ref = ref_fn()
    codes_g = Q.unpack_nibbles(_np(res.codes))
    codes_o = Q.unpack_nibbles(ref.codes)
    mismatch = np.mean(codes_g != codes_o)
    assert mismatch <= 1e-4, mismatch
    lg, lo = _np(res.block_loss), ref.block_loss
    assert np.all(np.abs(lg - lo) <= 1e-5 * np.maximum(lo, 1e-6 * lo.mean() + 1e-45))
    return ref


@pytest.mark.parametrize("n", [16, 32, 128])
def test_nvfp4_rotated(n):
    fq = _fp4()
    x = W.random_matrix(129, 2048, seed=70 + n, dist="laplace", dtype=torch.bfloat16)
    imp = W.random_importance(2048, seed=71)
    res = fq.quantize_nvfp4(x.to(DEV), imp.to(DEV), hadamard_n=n, check=True)
    torch.cuda.synchronize()
    ref = _rotated_checks(res, lambda: _oracle_nvfp4(x, imp, had=n), None, n)
    _check_nvfp4(res, ref)


@pytest.mark.parametrize("rows,cols", [(5, 2080), (130, 64)])
@pytest.mark.parametrize("window", [(-8, 8), (-16, 16)])
def test_mxfp4_fp32_wide_windows(rows, cols, window):
    """float32 input and windows of 17 and 33 exponents (the winner's codes
    are converted again rather than kept), MSE and WMSE."""
    fq = _fp4()
    x = W.random_matrix(rows, cols, seed=rows * cols, dist="t4", scale=0.3, dtype=torch.float32)
    r = fq.quantize_mxfp4(x.to(DEV), window=window, check=True)
    _check_mxfp4(r, Q.quantize_mxfp4(x.numpy(), window=window))
    imp = W.random_importance(cols, seed=cols + 3)
    r = fq.quantize_mxfp4(x.to(DEV), imp.to(DEV), window=window, check=True)
    _check_mxfp4(r, Q.quantize_mxfp4(x.numpy(), imp.numpy(), window=window))


@pytest.mark.parametrize("n", [16, 32, 64, 128])
def test_mxfp4_rotated(n):
    fq = _fp4()
    x = W.random_matrix(65, 4096, seed=80 + n, dist="laplace", scale=1.0, dtype=torch.bfloat16)
    res = fq.quantize_mxfp4(x.to(DEV), hadamard_n=n, check=True)
    torch.cuda.synchronize()
    ref = _rotated_checks(res, lambda: Q.quantize_mxfp4(_host_f32(x), hadamard_n=n), None, n)
    _check_mxfp4(res, ref)


# ------------------------------------------------- workload sizes ----
def _sample_rows(rows, k, seed):
    return np.sort(np.random.default_rng(seed).choice(rows, size=min(k, rows), replace=False))


def test_c1_nvfp4_mse_fp32_full():
    x = W.c1_weight()
    _check_nvfp4(_run_nvfp4(x), _oracle_nvfp4(x))


def test_c2_nvfp4_wmse_bf16_4096_sampled_rows():
    x, imp = W.c2_weight_and_importance()
    res = _run_nvfp4(x, imp)
    xf = _host_f32(x)
    S = Q.global_scale_nvfp4(xf)
    rows = _sample_rows(4096, 384, 202)
    ref = Q.quantize_nvfp4(xf[rows], imp.numpy(), global_scale=S)
    ref.global_scale = S
    _check_nvfp4(res, ref, rows=rows)


def test_tensor_beyond_2gib_sampled_rows():
    """65600 x 16384 bf16 (2.15 GB, past 2^31 bytes; 67 M blocks): NVFP4 WMSE
    (global-max pass + sweep) and MXFP4 checked bit-exact on rows on both
    sides of the 2^31-byte boundary.  The values are N(0, 0.02) clipped to
    +-0.5 with 0.75 planted in the last element, so the global maximum, and
    with it S, is known without reading the tensor back."""
    fq = _fp4()
    rows, cols = 65600, 16384
    g = torch.Generator(device=DEV)
    g.manual_seed(1201)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    for r0 in range(0, rows, 8192):
        r1 = min(rows, r0 + 8192)
        x[r0:r1] = (torch.randn((r1 - r0, cols), device=DEV, generator=g) * 0.02).clamp_(-0.5, 0.5).to(torch.bfloat16)
    x[-1, -1] = 0.75
    imp = W.random_importance(cols, seed=1202)
    pick = torch.tensor([0, 1, 32768, 65535, 65536, 65537, 65598, 65599], device=DEV)
    host = x[pick].float().cpu().numpy()
    S = Q.global_scale_nvfp4(np.array([[0.75]], np.float32))

    res = fq.quantize_nvfp4(x, imp.to(DEV), check=True)
    torch.cuda.synchronize()
    ref = Q.quantize_nvfp4(host, imp.numpy(), global_scale=S)
    _assert_equal("global_scale", np.float32(_np(res.global_scale)[0]), np.float32(S))
    for name, got, want in (("codes", res.codes, ref.codes), ("scales", res.scales, ref.scales),
                            ("offsets", res.offsets, ref.offsets), ("block_loss", res.block_loss, ref.block_loss)):
        _assert_equal(name, _np(got[pick]), want)
    del res

    mx = fq.quantize_mxfp4(x, window=(-1, 0), check=True)
    torch.cuda.synchronize()
    mref = Q.quantize_mxfp4(host, window=(-1, 0))
    for name, got, want in (("codes", mx.codes, mref.codes), ("scales", mx.scales, mref.scales),
                            ("offsets", mx.offsets, mref.offsets), ("block_loss", mx.block_loss, mref.block_loss)):
        _assert_equal("mxfp4 " + name, _np(got[pick]), want)


@pytest.mark.parametrize("variant", ["absmax", "sweep", "rot32"])
def test_c3_mxfp4_activations_sampled_rows(variant):
    fq = _fp4()
    x = W.c3_activation()
    window = (0, 0) if variant == "absmax" else (-1, 0)
    had = 32 if variant == "rot32" else 0
    res = fq.quantize_mxfp4(x.to(DEV), window=window, hadamard_n=had, check=True)
    torch.cuda.synchronize()
    rows = _sample_rows(8192, 256, 303)
    ref = Q.quantize_mxfp4(_host_f32(x[rows]), window=window, hadamard_n=had)
    _check_mxfp4(res, ref, rows=rows)


@pytest.mark.parametrize("name", list(W.LAYER_8B))
def test_c4_8b_layer_sampled_rows(name):
    x = W.c4_matrix(name)
    imp = W.c4_importance(name)
    xf = _host_f32(x)
    S = Q.global_scale_nvfp4(xf)
    rows = _sample_rows(x.shape[0], 96, 404)
    for im in (None, imp):
        res = _run_nvfp4(x, im)
        ref = Q.quantize_nvfp4(xf[rows], None if im is None else im.numpy(), global_scale=S)
        _check_nvfp4(res, ref, rows=rows)


@pytest.mark.parametrize("name", list(W.LAYER_70B))
def test_c5_70b_layer0_rotated_sampled_rows(name):
    fq = _fp4()
    x = W.c5_matrix(0, name, DEV)
    imp = W.c5_importance(name)
    res = fq.quantize_nvfp4(x, imp.to(DEV), hadamard_n=16, check=True)
    torch.cuda.synchronize()
    xf = _host_f32(x)
    del x
    # S from the oracle's own rotation of the whole matrix, row chunk by row chunk
    amax = np.float32(0)
    for r0 in range(0, xf.shape[0], 1024):
        amax = max(amax, np.abs(OH.block_hadamard(xf[r0:r0 + 1024], 16)).max())
    S = np.float32(np.float32(amax) / np.float32(1536))
    rows = _sample_rows(xf.shape[0], 64, 505)
    ref = Q.quantize_nvfp4(xf[rows], imp.numpy(), global_scale=S, hadamard_n=16)
    ref.global_scale = S
    _check_nvfp4(res, ref, rows=rows)


# --------------------------------------------------- FOCUS quantizer ----
@pytest.mark.parametrize("fmt,sub", [("nvfp4", 4), ("nvfp4", 8), ("nvfp4", 16),
                                     ("mxfp4", 4), ("mxfp4", 8), ("mxfp4", 16), ("mxfp4", 32)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_relaxed_quantizer(fmt, sub, dtype):
    fq = _fp4()
    rows, cols = 67, 2080
    x = W.random_matrix(rows, cols, seed=90 + sub, dist="t4", dtype=dtype)
    xd = x.to(DEV)
    if fmt == "nvfp4":
        base = fq.quantize_nvfp4(xd)
        gs = base.global_scale
    else:
        base = fq.quantize_mxfp4(xd)
        gs = None
    c = torch.from_numpy(np.exp(np.random.default_rng(sub).normal(0, 0.2, (rows, cols // sub)))).to(torch.float16)
    codes, dq = fq.quantize_relaxed(xd, base.scales, c.to(DEV), fmt=fmt, global_scale=gs, sub=sub, check=True)
    torch.cuda.synchronize()
    ref_codes, ref_dq = FO.quantize_given_scales(_host_f32(x), fmt, _np(base.scales),
                                                 None if gs is None else _np(gs)[0], c.numpy(), sub=sub)
    _assert_equal("relaxed codes", _np(codes), ref_codes)
    _assert_equal("relaxed dequant", _np(dq), ref_dq)
    # unit coefficients reproduce the scale search's own codes
    codes1, _ = fq.quantize_relaxed(xd, base.scales, None, fmt=fmt, global_scale=gs, sub=sub, dequant=False,
                                    check=True)
    torch.cuda.synchronize()
    _assert_equal("relaxed c=1 vs sweep codes", _np(codes1), _np(base.codes))


def test_relaxed_quantizer_data_errors():
    fq = _fp4()
    x = W.random_matrix(4, 64, seed=98).to(DEV)
    base = fq.quantize_nvfp4(x)
    bad = base.scales.clone()
    bad[1, 2] = 0
    with pytest.raises(fq.FP4QError, match="scale or coefficient"):
        fq.quantize_relaxed(x, bad, None, global_scale=base.global_scale, check=True)
    c = torch.ones(4, 8, dtype=torch.float16, device=DEV)
    c[0, 3] = -1.0
    with pytest.raises(fq.FP4QError, match="scale or coefficient"):
        fq.quantize_relaxed(x, base.scales, c, global_scale=base.global_scale, check=True)
    fq.quantize_relaxed(x, base.scales, None, global_scale=base.global_scale, check=True)


# ------------------------------------------------------ scale study ----
def test_study_histogram_and_rule_ordering():
    from fp4_post_quantization_amd import study
    fq = _fp4()
    x = W.random_matrix(96, 1024, seed=99, dist="laplace", dtype=torch.bfloat16)
    xd = x.to(DEV)
    r = fq.quantize_mxfp4(xd, hadamard_n=32)
    ref = Q.quantize_mxfp4(_host_f32(x), hadamard_n=32)
    h = study.code_histogram(r.codes).cpu().numpy()
    np.testing.assert_array_equal(h, np.bincount(Q.unpack_nibbles(ref.codes).ravel(), minlength=16))
    imp = W.random_importance(1024, seed=100).to(DEV)
    res = study.nvfp4_scale_rules(xd, imp, iters=2)
    a = fq.quantize_nvfp4(xd, imp, window=(0, 0)).block_loss
    s_ = fq.quantize_nvfp4(xd, imp, window=(-8, 7)).block_loss
    e = fq.quantize_nvfp4(xd, imp, window=(-126, 126)).block_loss
    torch.cuda.synchronize()
    # wider windows contain the narrower ones and use identical arithmetic
    assert bool((s_ <= a).all()) and bool((e <= s_).all())
    assert res["sweep_vs_absmax"]["loss_reduction"] >= 0
    assert res["exhaustive_vs_sweep"]["loss_reduction"] >= 0
    assert sum(res["sweep_offset_histogram"].values()) == res["blocks"]
    u = study.mxfp4_code_usage(xd, window=(0, 0))
    assert abs(sum(u["magnitude_histogram"]) - x.numel()) == 0


# ------------------------------------------------------------- GPTQ ----
def _gptq_inputs(rows, cols, seed):
    w = W.random_matrix(rows, cols, seed=seed, dist="t4")
    X = W.calibration_activations(4 * cols, cols, seed=seed + 1)
    H, U = W.hessian_and_factor(X)
    imp = torch.from_numpy(np.diag(H).astype(np.float32))
    return w, H, U, imp


@pytest.mark.parametrize("wmse", [False, True])
def test_gptq_single_batch_bitexact(wmse):
    """One 128-column batch involves no contraction, so GPU and oracle
    follow the same float32 steps: codes, scales and S are bit-exact."""
    fq = _fp4()
    w, H, U, imp = _gptq_inputs(37, 128, seed=110)
    im = imp if wmse else None
    res = fq.gptq_nvfp4(w.to(DEV), U, None if im is None else im.to(DEV), check=True)
    torch.cuda.synchronize()
    codes, scales, S = GQ.gptq_nvfp4(w.numpy(), U, None if im is None else im.numpy())
    _assert_equal("gptq S", np.float32(_np(res.global_scale)[0]), S)
    _assert_equal("gptq scales", _np(res.scales), scales)
    _assert_equal("gptq codes", _np(res.codes), codes)


def test_gptq_without_feedback_equals_sweep():
    fq = _fp4()
    w = W.random_matrix(64, 512, seed=111, dist="t4").to(DEV)
    U = np.diag(np.exp(np.random.default_rng(112).normal(0, 0.3, 512))).astype(np.float32)
    imp = W.random_importance(512, seed=113).to(DEV)
    for im in (None, imp):
        g = fq.gptq_nvfp4(w, U, im, check=True)
        s_ = fq.quantize_nvfp4(w, im, check=True)
        torch.cuda.synchronize()
        _assert_equal("codes", _np(g.codes), _np(s_.codes))
        _assert_equal("scales", _np(g.scales), _np(s_.scales))


@pytest.mark.parametrize("wmse", [False, True])
@pytest.mark.parametrize("rows,cols", [(192, 512), (96, 768)])
def test_gptq_multi_batch_against_oracle(wmse, rows, cols):
    """Across batches the trailing update is an MFMA contraction whose
    summation order differs from the oracle's float64 product, so values
    agree to float32 rounding: code and scale mismatch rates <= 1e-3, GPTQ
    proxy losses within 1e-3 relative, and both below round-to-nearest.
    768 columns: a block of six batches, where the update after the fourth
    (four batches' errors onto the next four) is cut to the two left."""
    fq = _fp4()
    w, H, U, imp = _gptq_inputs(rows, cols, seed=114 + cols - 512)
    im = imp if wmse else None
    res = fq.gptq_nvfp4(w.to(DEV), U, None if im is None else im.to(DEV), check=True)
    torch.cuda.synchronize()
    codes, scales, S = GQ.gptq_nvfp4(w.numpy(), U, None if im is None else im.numpy())
    gc, gs = _np(res.codes), _np(res.scales)
    assert np.float32(_np(res.global_scale)[0]) == S
    assert np.mean(Q.unpack_nibbles(gc) != Q.unpack_nibbles(codes)) <= 1e-3
    assert np.mean(gs != scales) <= 1e-3
    lg = GQ.proxy_loss(w.numpy(), gc, gs, S, H)
    lo = GQ.proxy_loss(w.numpy(), codes, scales, S, H)
    rtn = Q.quantize_nvfp4(w.numpy(), None if im is None else im.numpy())
    lr = GQ.proxy_loss(w.numpy(), rtn.codes, rtn.scales, rtn.global_scale, H)
    assert abs(lg - lo) <= 1e-3 * lo
    assert lg < lr and lo < lr


@pytest.mark.parametrize("rows,cols,wmse", [(64, 2304, False), (200, 2176, True)])
def test_gptq_block_updates_against_oracle(rows, cols, wmse):
    """Past 1024 columns: each full 1024-column block's errors reach the later
    columns as one contraction (on the bf16 matrix cores with operands split
    in three), then the tail.  2304 columns: two blocks and a 256-column
    tail; 2176: two blocks and a 128-column tail, on 200 rows (one full and
    one ragged 128-row tile).  Same bar as the multi-batch case."""
    fq = _fp4()
    w, H, U, imp = _gptq_inputs(rows, cols, seed=116 + rows)
    im = imp if wmse else None
    res = fq.gptq_nvfp4(w.to(DEV), U, None if im is None else im.to(DEV), check=True)
    torch.cuda.synchronize()
    codes, scales, S = GQ.gptq_nvfp4(w.numpy(), U, None if im is None else im.numpy())
    gc, gs = _np(res.codes), _np(res.scales)
    assert np.float32(_np(res.global_scale)[0]) == S
    code_mis = np.mean(Q.unpack_nibbles(gc) != Q.unpack_nibbles(codes))
    scale_mis = np.mean(gs != scales)
    lg = GQ.proxy_loss(w.numpy(), gc, gs, S, H)
    lo = GQ.proxy_loss(w.numpy(), codes, scales, S, H)
    print(f"code mismatch {code_mis:.2e}, scale mismatch {scale_mis:.2e}, loss rel {abs(lg - lo) / lo:.2e}")
    assert code_mis <= 1e-3 and scale_mis <= 1e-3
    assert abs(lg - lo) <= 1e-3 * lo


def test_gptq_reads_the_weight_in_place_of_a_copy():
    """A float32 weight is read where it lies (each column until an update
    first writes the working storage) and left unchanged; the results are
    bit-identical to a call on a working copy holding the weight (w_in NULL),
    for both formats, over 2304 columns (first touches by the first batch,
    the block's updates and the far update) on a ragged 200 rows."""
    fq = _fp4()
    from fp4_post_quantization_amd import _lib as L
    lib = L.load()
    w, H, U, imp = _gptq_inputs(200, 2304, seed=131)
    wd, Ud, imd = w.to(DEV), torch.from_numpy(U).to(DEV), imp.to(DEV)
    before = wd.clone()
    rows, cols = wd.shape
    ws = torch.zeros(lib.fp4q_workspace_bytes(), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    nv = fq.gptq_nvfp4(wd, Ud, imd, check=True)
    work = wd.clone()
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=DEV)
    gs = torch.empty(1, dtype=torch.float32, device=DEV)
    L.check(lib.fp4q_gptq_nvfp4(work.data_ptr(), rows, cols, cols, None, 0, Ud.data_ptr(), imd.data_ptr(), -8, 7,
                                0, codes.data_ptr(), scales.data_ptr(), gs.data_ptr(), ws.data_ptr(), ws.numel(),
                                stream))
    mx = fq.gptq_mxfp4(wd, Ud, imd, check=True)
    work2 = wd.clone()
    mcodes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV)
    mscales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    L.check(lib.fp4q_gptq_mxfp4(work2.data_ptr(), rows, cols, cols, None, 0, Ud.data_ptr(), imd.data_ptr(), -1, 0,
                                mcodes.data_ptr(), mscales.data_ptr(), ws.data_ptr(), ws.numel(), stream))
    # a weight with a wider row stride (a column slice) is read in place as well
    wide = torch.zeros((rows, cols + 64), dtype=torch.float32, device=DEV)
    wide[:, :cols] = wd
    nvs = fq.gptq_nvfp4(wide[:, :cols], Ud, imd, check=True)
    torch.cuda.synchronize()
    assert torch.equal(wd, before), "the weight was written"
    assert torch.equal(wide[:, :cols], before), "the strided weight was written"
    _assert_equal("nvfp4 codes, strided weight", _np(nvs.codes), _np(nv.codes))
    _assert_equal("nvfp4 scales, strided weight", _np(nvs.scales), _np(nv.scales))
    _assert_equal("nvfp4 codes", _np(nv.codes), _np(codes))
    _assert_equal("nvfp4 scales", _np(nv.scales), _np(scales))
    _assert_equal("nvfp4 S", _np(nv.global_scale), _np(gs))
    _assert_equal("mxfp4 codes", _np(mx.codes), _np(mcodes))
    _assert_equal("mxfp4 scales", _np(mx.scales), _np(mscales))


@pytest.mark.parametrize("wmse", [False, True])
def test_gptq_mxfp4_single_batch_bitexact(wmse):
    """MXFP4 GPTQ, one batch (no contraction): bit-exact codes and exponents."""
    fq = _fp4()
    w, H, U, imp = _gptq_inputs(37, 128, seed=120)
    im = imp if wmse else None
    for window in ((-1, 0), (-2, 1)):
        res = fq.gptq_mxfp4(w.to(DEV), U, None if im is None else im.to(DEV), window=window, check=True)
        torch.cuda.synchronize()
        codes, scales = GQ.gptq_mxfp4(w.numpy(), U, None if im is None else im.numpy(), window=window)
        _assert_equal("gptq_mx scales", _np(res.scales), scales)
        _assert_equal("gptq_mx codes", _np(res.codes), codes)


def test_gptq_mxfp4_without_feedback_equals_sweep():
    fq = _fp4()
    w = W.random_matrix(64, 512, seed=121, dist="t4").to(DEV)
    U = np.diag(np.exp(np.random.default_rng(122).normal(0, 0.3, 512))).astype(np.float32)
    imp = W.random_importance(512, seed=123).to(DEV)
    for im in (None, imp):
        g = fq.gptq_mxfp4(w, U, im, check=True)
        s_ = fq.quantize_mxfp4(w, im, check=True)
        torch.cuda.synchronize()
        _assert_equal("codes", _np(g.codes), _np(s_.codes))
        _assert_equal("scales", _np(g.scales), _np(s_.scales))


@pytest.mark.parametrize("rows,cols,wmse", [(192, 512, False), (192, 512, True), (96, 768, True),
                                             (64, 2304, False), (200, 2176, True)])
def test_gptq_mxfp4_multi_batch_against_oracle(rows, cols, wmse):
    """MXFP4 GPTQ across batches (and, at 2304 columns, across 1024-column
    blocks): the same bar as NVFP4 GPTQ."""
    fq = _fp4()
    w, H, U, imp = _gptq_inputs(rows, cols, seed=124 + cols)
    im = imp if wmse else None
    res = fq.gptq_mxfp4(w.to(DEV), U, None if im is None else im.to(DEV), check=True)
    torch.cuda.synchronize()
    codes, scales = GQ.gptq_mxfp4(w.numpy(), U, None if im is None else im.numpy())
    gc, gs = _np(res.codes), _np(res.scales)
    assert np.mean(Q.unpack_nibbles(gc) != Q.unpack_nibbles(codes)) <= 1e-3
    assert np.mean(gs != scales) <= 1e-3
    lg = GQ.proxy_loss_mx(w.numpy(), gc, gs, H)
    lo = GQ.proxy_loss_mx(w.numpy(), codes, scales, H)
    rtn = Q.quantize_mxfp4(w.numpy(), None if im is None else im.numpy())
    lr = GQ.proxy_loss_mx(w.numpy(), rtn.codes, rtn.scales, H)
    assert abs(lg - lo) <= 1e-3 * lo
    assert lg < lr and lo < lr


def test_gptq_data_errors_set_status():
    fq = _fp4()
    w, H, U, imp = _gptq_inputs(8, 128, seed=130)
    bad_w = w.clone()
    bad_w[3, 17] = float("nan")
    with pytest.raises(fq.FP4QError, match="non-finite"):
        fq.gptq_mxfp4(bad_w.to(DEV), U, check=True)
    with pytest.raises(fq.FP4QError, match="non-finite"):
        fq.gptq_nvfp4(bad_w.to(DEV), U, check=True)
    bad_imp = imp.clone()
    bad_imp[5] = -1.0
    with pytest.raises(fq.FP4QError, match="importance"):
        fq.gptq_mxfp4(w.to(DEV), U, bad_imp.to(DEV), check=True)
    with pytest.raises(fq.FP4QError, match="importance"):
        fq.gptq_nvfp4(w.to(DEV), U, bad_imp.to(DEV), check=True)


def test_gptq_given_scale_data_errors_set_status():
    """With a given global scale no max pass reads the weights: the batch
    kernel flags non-finite weights, the call's first kernel an invalid S."""
    fq = _fp4()
    w, H, U, imp = _gptq_inputs(8, 128, seed=131)
    S = float(np.abs(w.numpy()).max()) / 1536
    bad_w = w.clone()
    bad_w[5, 100] = float("inf")
    with pytest.raises(fq.FP4QError, match="non-finite"):
        fq.gptq_nvfp4(bad_w.to(DEV), U, global_scale=S, check=True)
    for bad_s in (float("nan"), -1.0, float("inf")):
        with pytest.raises(fq.FP4QError, match="global scale"):
            fq.gptq_nvfp4(w.to(DEV), U, global_scale=bad_s, check=True)
    ok = fq.gptq_nvfp4(w.to(DEV), U, global_scale=S, check=True)
    ref = fq.gptq_nvfp4(w.to(DEV), U, check=True)
    if np.float32(S) == np.float32(_np(ref.global_scale)[0]):
        assert torch.equal(ok.codes, ref.codes) and torch.equal(ok.scales, ref.scales)


def test_status_word_belongs_to_the_last_call():
    """Every call writes the workspace's status word on its stream before
    any kernel can set a bit: a workspace full of garbage reports no error
    for clean data, and an error does not outlive its call."""
    fq = _fp4()
    x = W.random_matrix(16, 256, seed=57).to(DEV)
    imp = W.random_importance(256, seed=58).to(DEV)
    bad = x.clone()
    bad[2, 5] = float("nan")
    U = torch.eye(128)
    calls = [
        lambda ws, t: fq.quantize_nvfp4(t, imp, ws=ws),
        lambda ws, t: fq.quantize_nvfp4(t, imp, global_scale=0.01, ws=ws),
        lambda ws, t: fq.quantize_mxfp4(t, imp, ws=ws),
        lambda ws, t: fq.gptq_nvfp4(t[:, :128], U, ws=ws),
        lambda ws, t: fq.gptq_mxfp4(t[:, :128], U, ws=ws),
        lambda ws, t: fq.global_scale_nvfp4(t, ws=ws),
    ]
    for k, call in enumerate(calls):
        ws = torch.full((fq.workspace(DEV).numel(),), 0xFF, dtype=torch.uint8, device=DEV)
        call(ws, x)
        torch.cuda.synchronize()
        assert fq.read_status(ws) == 0, k
        call(ws, bad)
        torch.cuda.synchronize()
        assert fq.read_status(ws) & 0x1, k
        call(ws, x)
        torch.cuda.synchronize()
        assert fq.read_status(ws) == 0, k
    # FP4Q_ACCUMULATE_STATUS: errors add up over a chain of calls, and a given scale or the
    # importance are still validated (by the sweep itself)
    ws = torch.zeros(fq.workspace(DEV).numel(), dtype=torch.uint8, device=DEV)
    S = fq.quantize_nvfp4(x, imp, ws=ws).global_scale
    fq.quantize_nvfp4(bad, imp, ws=ws, accumulate_status=True)
    fq.quantize_nvfp4(x, imp, global_scale=S, ws=ws, accumulate_status=True)
    torch.cuda.synchronize()
    assert fq.read_status(ws) == 0x1
    bad_imp = imp.clone()
    bad_imp[7] = -2.0
    fq.quantize_nvfp4(x, bad_imp, global_scale=S, ws=ws, accumulate_status=True)
    fq.quantize_nvfp4(x, imp, global_scale=float("nan"), ws=ws, accumulate_status=True)
    torch.cuda.synchronize()
    assert fq.read_status(ws) == 0x7
    a = fq.quantize_nvfp4(x, imp, global_scale=S, ws=ws, accumulate_status=True)
    b = fq.quantize_nvfp4(x, imp, global_scale=S)
    for f in ("codes", "scales", "block_loss", "offsets"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    # the slot's tag (bytes 4..7) is the dispatch ID of each call's first kernel: it changes per call
    ws = torch.zeros(fq.workspace(DEV).numel(), dtype=torch.uint8, device=DEV)
    tags = []
    for _ in range(3):
        fq.quantize_mxfp4(x, ws=ws)
        torch.cuda.synchronize()
        tags.append(int(ws[4:8].view(torch.int32).item()))
    assert len(set(tags)) == 3 and fq.read_status(ws) == 0
    # empty tensors clear it too
    ws = torch.full((fq.workspace(DEV).numel(),), 0xFF, dtype=torch.uint8, device=DEV)
    fq.quantize_nvfp4(x[:0], ws=ws)
    fq.quantize_mxfp4(x[:0], ws=ws)
    torch.cuda.synchronize()
    assert fq.read_status(ws) == 0


def test_gptq_bad_hessian_sets_status():
    fq = _fp4()
    w = W.random_matrix(8, 128, seed=115).to(DEV)
    U = np.eye(128, dtype=np.float32)
    U[5, 5] = 0.0
    with pytest.raises(fq.FP4QError, match="inverse-Hessian"):
        fq.gptq_nvfp4(w, U, check=True)


# ------------------------------------------- the layer stream's records ----
def test_c5_stream_checksums_and_resume(tmp_path):
    """The 70B-shaped stream on small shapes: three layers in one run give
    the same per-layer checksums and stream digest as two layers followed by
    a run resumed at layer 2 from the state file, and as a run with each
    layer's calls on two streams; resuming without the
    earlier layers' records is refused; the device checksum equals a host
    recomputation."""
    import bench
    shapes = {"q": (64, 256), "k": (32, 256), "down": (256, 512)}
    imps = {n: W.random_importance(c, seed=600 + c).to(DEV) for n, (r, c) in shapes.items()}
    full = bench.c5_stream(3, imps, state_path=str(tmp_path / "a.json"), shapes=shapes)
    bench.c5_stream(2, imps, state_path=str(tmp_path / "b.json"), shapes=shapes)
    resumed = bench.c5_stream(3, imps, start_layer=2, state_path=str(tmp_path / "b.json"), shapes=shapes)
    assert resumed["stream_digest"] == full["stream_digest"] and resumed["records"] == 3
    # the calls of each layer spread over two streams: the same records
    two = bench.c5_stream(3, imps, shapes=shapes, streams=2)
    assert two["stream_digest"] == full["stream_digest"] and two["records"] == 3
    assert json.load(open(tmp_path / "a.json")) == json.load(open(tmp_path / "b.json"))
    with pytest.raises(SystemExit):
        bench.c5_stream(3, imps, start_layer=2, state_path=str(tmp_path / "missing.json"), shapes=shapes)
    codes = torch.randint(0, 256, (64, 128), dtype=torch.uint8)
    words = codes.numpy().reshape(-1).view(np.uint32).astype(object)
    host = sum((i + 1) * int(w) for i, w in enumerate(words)) % 2**63
    assert bench._digest(codes.to(DEV)) == host


# ------------------------------------------------ GPTQ, static reordering ----
def _gptq_static_inputs(rows, cols, seed):
    w = W.random_matrix(rows, cols, seed=seed, dist="t4")
    X = W.calibration_activations(4 * cols, cols, seed=seed + 1)
    H, perm, U = W.act_order_and_factor(X)
    imp = torch.from_numpy(np.diag(H).astype(np.float32))
    return w, H, perm, U, imp


def _static_call(fmt, w, perm, U, im, **kw):
    fq = _fp4()
    f = fq.gptq_static_nvfp4 if fmt == "nvfp4" else fq.gptq_static_mxfp4
    return f(w.to(DEV), torch.from_numpy(perm).to(DEV), U, None if im is None else im.to(DEV), check=True, **kw)


def _static_oracle(fmt, w, perm, U, im, **kw):
    f = GQ.gptq_nvfp4_static if fmt == "nvfp4" else GQ.gptq_mxfp4_static
    return f(w.numpy(), U, perm, None if im is None else im.numpy(), **kw)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("wmse", [False, True])
def test_gptq_static_single_batch_bitexact(fmt, wmse):
    """Static reordering, one 128-column batch (no contraction): the scales
    come from the sweep on the weight as given and each processing slot is
    rounded at its stored group's scale, in the oracle's float32 steps:
    codes (back in the stored order), scales and S are bit-exact."""
    w, H, perm, U, imp = _gptq_static_inputs(37, 128, seed=140)
    im = imp if wmse else None
    res = _static_call(fmt, w, perm, U, im)
    torch.cuda.synchronize()
    ref = _static_oracle(fmt, w, perm, U, im)
    if fmt == "nvfp4":
        _assert_equal("static S", np.float32(_np(res.global_scale)[0]), ref[2])
    _assert_equal("static scales", _np(res.scales), ref[1])
    _assert_equal("static codes", _np(res.codes), ref[0])


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_gptq_static_without_feedback_equals_sweep(fmt):
    """A diagonal factor moves no error: whatever the order, the result is
    the plain quantizer's, bit for bit (MSE and WMSE)."""
    fq = _fp4()
    w = W.random_matrix(64, 512, seed=141, dist="t4")
    U = np.diag(np.exp(np.random.default_rng(142).normal(0, 0.3, 512))).astype(np.float32)
    perm = np.random.default_rng(143).permutation(512).astype(np.int32)
    imp = W.random_importance(512, seed=144)
    for im in (None, imp):
        g = _static_call(fmt, w, perm, U, im)
        q = (fq.quantize_nvfp4 if fmt == "nvfp4" else fq.quantize_mxfp4)(
            w.to(DEV), None if im is None else im.to(DEV), check=True)
        torch.cuda.synchronize()
        _assert_equal("codes", _np(g.codes), _np(q.codes))
        _assert_equal("scales", _np(g.scales), _np(q.scales))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("rows,cols,wmse", [(192, 512, False), (96, 768, True), (200, 2176, True)])
def test_gptq_static_multi_batch_against_oracle(fmt, rows, cols, wmse):
    """Static reordering across batches and (2176 columns) 1024-column
    blocks: the scales are fixed before any update, so they are bit-exact;
    codes differ from the oracle's float64 trailing product by float32
    rounding only (mismatch <= 1e-3), proxy losses agree within 1e-3 and lie
    below round-to-nearest."""
    w, H, perm, U, imp = _gptq_static_inputs(rows, cols, seed=145 + cols)
    im = imp if wmse else None
    res = _static_call(fmt, w, perm, U, im)
    torch.cuda.synchronize()
    ref = _static_oracle(fmt, w, perm, U, im)
    gc, gs = _np(res.codes), _np(res.scales)
    _assert_equal("static scales", gs, ref[1])
    mis = np.mean(Q.unpack_nibbles(gc) != Q.unpack_nibbles(ref[0]))
    if fmt == "nvfp4":
        S = ref[2]
        assert np.float32(_np(res.global_scale)[0]) == S
        lg, lo = GQ.proxy_loss(w.numpy(), gc, gs, S, H), GQ.proxy_loss(w.numpy(), ref[0], ref[1], S, H)
        rtn = Q.quantize_nvfp4(w.numpy(), None if im is None else im.numpy())
        lr = GQ.proxy_loss(w.numpy(), rtn.codes, rtn.scales, rtn.global_scale, H)
    else:
        lg, lo = GQ.proxy_loss_mx(w.numpy(), gc, gs, H), GQ.proxy_loss_mx(w.numpy(), ref[0], ref[1], H)
        rtn = Q.quantize_mxfp4(w.numpy(), None if im is None else im.numpy())
        lr = GQ.proxy_loss_mx(w.numpy(), rtn.codes, rtn.scales, H)
    print(f"code mismatch {mis:.2e}, loss rel {abs(lg - lo) / lo:.2e}, vs round-to-nearest {lg / lr:.3f}")
    assert mis <= 1e-3
    assert abs(lg - lo) <= 1e-3 * lo
    assert lg < lr


def test_gptq_static_full_size_sampled_rows():
    """4096 x 4096 (the GPTQ bench's shape), NVFP4 MSE with act-order: rows
    are independent under GPTQ, so the oracle runs on 24 sampled rows with
    the same factor and S; scales bit-exact, codes within the multi-batch
    bar."""
    rows = cols = 4096
    w = W.random_matrix(rows, cols, seed=150, dist="t4")
    X = W.calibration_activations(2048, cols, seed=151)
    H, perm, U = W.act_order_and_factor(X)
    res = _static_call("nvfp4", w, perm, U, None)
    torch.cuda.synchronize()
    S = np.float32(_np(res.global_scale)[0])
    assert S == Q.global_scale_nvfp4(w.numpy())
    pick = np.sort(np.random.default_rng(152).choice(rows, 24, replace=False))
    codes, scales, _ = GQ.gptq_nvfp4_static(w.numpy()[pick], U, perm, global_scale=S)
    _assert_equal("static scales (sampled rows)", _np(res.scales)[pick], scales)
    mis = np.mean(Q.unpack_nibbles(_np(res.codes)[pick]) != Q.unpack_nibbles(codes))
    print(f"code mismatch on sampled rows {mis:.2e}")
    assert mis <= 1e-3


def test_gptq_static_bad_order_sets_status():
    """A repeated or out-of-range entry in the order is reported (entries
    are clamped, so nothing is read out of bounds); a valid call afterwards
    on the same data is exact again."""
    fq = _fp4()
    w, H, perm, U, imp = _gptq_static_inputs(8, 128, seed=153)
    dup = perm.copy()
    dup[7] = dup[3]
    oob = perm.copy()
    oob[11] = 128
    neg = perm.copy()
    neg[0] = -5
    for bad in (dup, oob, neg):
        for fmt in ("nvfp4", "mxfp4"):
            with pytest.raises(fq.FP4QError, match="permutation"):
                _static_call(fmt, w, bad, U, None)
    res = _static_call("nvfp4", w, perm, U, None)
    torch.cuda.synchronize()
    ref = _static_oracle("nvfp4", w, perm, U, None)
    _assert_equal("static codes after bad calls", _np(res.codes), ref[0])


# ------------------------------------------------------- calls on streams ----
def test_calls_on_two_streams_match_one_stream():
    """The library keeps no state between calls: quantize calls of several
    matrices issued alternately on two HIP streams (each stream its own
    workspace and outputs, the bench's pipelined steps), and GPTQ calls
    likewise, give bit for bit what the same calls give one after another,
    and every status word stays clear."""
    fq = _fp4()
    xs = [W.random_matrix(512, 1024, seed=160 + j, dist="t4").to(DEV).to(torch.bfloat16) for j in range(4)]
    imp = W.random_importance(1024, seed=165).to(DEV)
    ref = [fq.quantize_nvfp4(x, imp, check=True) for x in xs]
    mref = [fq.quantize_mxfp4(x, window=(-1, 0), hadamard_n=32, check=True) for x in xs]
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    wss = [torch.zeros_like(fq.workspace(DEV)) for _ in streams]
    got, mgot = [], []
    for rep in range(3):
        for j, x in enumerate(xs):
            k = (rep * len(xs) + j) % 2
            with torch.cuda.stream(streams[k]):
                got.append((j, fq.quantize_nvfp4(x, imp, ws=wss[k])))
                mgot.append((j, fq.quantize_mxfp4(x, window=(-1, 0), hadamard_n=32, ws=wss[k])))
    torch.cuda.synchronize()
    for j, r in got:
        for f in ("codes", "scales", "global_scale", "block_loss", "offsets"):
            assert torch.equal(getattr(r, f), getattr(ref[j], f)), (j, f)
    for j, r in mgot:
        assert torch.equal(r.codes, mref[j].codes) and torch.equal(r.scales, mref[j].scales), j
    assert [fq.read_status(w) for w in wss] == [0, 0]

    w, H, U, imp_g = _gptq_inputs(96, 512, seed=166)
    ws_ = [w.to(DEV), (w * 0.5).to(DEV), (-w).to(DEV)]
    gref = [fq.gptq_nvfp4(m, U) for m in ws_]
    gout = []
    for i in range(6):
        with torch.cuda.stream(streams[i % 2]):
            gout.append((i % 3, fq.gptq_nvfp4(ws_[i % 3], U)))
    torch.cuda.synchronize()
    for j, r in gout:
        assert torch.equal(r.codes, gref[j].codes) and torch.equal(r.scales, gref[j].scales), j


def test_gptq_static_given_scale_and_empty():
    """Static reordering with the global scale given: passing back the scale
    the call computed gives the same codes and scales, a NaN scale is
    reported, and an empty matrix returns empty results without errors."""
    fq = _fp4()
    w, H, perm, U, imp = _gptq_static_inputs(24, 256, seed=170)
    a = _static_call("nvfp4", w, perm, U, imp)
    b = _static_call("nvfp4", w, perm, U, imp, global_scale=float(_np(a.global_scale)[0]))
    torch.cuda.synchronize()
    for f in ("codes", "scales", "global_scale"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    with pytest.raises(fq.FP4QError, match="global scale"):
        _static_call("nvfp4", w, perm, U, imp, global_scale=float("nan"))
    e = fq.gptq_static_nvfp4(torch.zeros((0, 256), device=DEV), torch.from_numpy(perm).to(DEV), U, check=True)
    m = fq.gptq_static_mxfp4(torch.zeros((0, 256), device=DEV), torch.from_numpy(perm).to(DEV), U, check=True)
    torch.cuda.synchronize()
    assert e.codes.shape == (0, 128) and e.scales.shape == (0, 16) and m.scales.shape == (0, 8)

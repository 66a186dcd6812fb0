"""fp4q_quantize_nvfp4_noalloc (no workspace, static device scratch) against
fp4q_quantize_nvfp4 through the C ABI: identical codes, scales, offsets,
losses and global scale, on two calls in a row (the second on a smaller
input), the status output, and replays of a captured HIP graph."""

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _fq():
    import fp4_post_quantization_amd as fq
    return fq


def _empty_result(fq, rows, cols):
    return fq.NVFP4Result(
        codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV),
        scales=torch.empty((rows, cols // 16), dtype=torch.uint8, device=DEV),
        global_scale=torch.empty(1, dtype=torch.float32, device=DEV),
        block_loss=torch.empty((rows, cols // 16), dtype=torch.float32, device=DEV),
        offsets=torch.empty((rows, cols // 16), dtype=torch.int8, device=DEV))


def _assert_same(a, b):
    for f in ("codes", "scales", "global_scale", "block_loss", "offsets"):
        x, y = getattr(a, f), getattr(b, f)
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), f


@pytest.mark.parametrize("dtype,had,wmse", [(torch.bfloat16, 0, True), (torch.float32, 0, False),
                                            (torch.bfloat16, 16, True), (torch.float32, 128, False)])
def test_noalloc_matches_workspace_call_twice(dtype, had, wmse):
    fq = _fq()
    status = torch.full((2,), -1, dtype=torch.int32, device=DEV)   # garbage: the call writes it
    for rows, cols, seed in ((300, 4096, 1), (37, 1024, 2)):       # the second call is smaller
        x = W.random_matrix(rows, cols, seed=seed, dist="t4", dtype=dtype).to(DEV)
        imp = W.random_importance(cols, seed=seed + 10).to(DEV) if wmse else None
        ref = fq.quantize_nvfp4(x, imp, hadamard_n=had, check=True)
        out = _empty_result(fq, rows, cols)
        before = torch.cuda.memory_allocated()
        fq.quantize_nvfp4_noalloc(x, imp, hadamard_n=had, out=out, status=status)
        assert torch.cuda.memory_allocated() == before
        torch.cuda.synchronize()
        _assert_same(out, ref)
        assert int(status[0].item()) == 0
        # with the scale given
        out2 = _empty_result(fq, rows, cols)
        out2.global_scale.copy_(ref.global_scale)
        fq.quantize_nvfp4_noalloc(x, imp, hadamard_n=had, out=out2, status=status, given_scale=True)
        torch.cuda.synchronize()
        _assert_same(out2, ref)
        assert int(status[0].item()) == 0


def test_noalloc_status_and_scratch_size():
    fq = _fq()
    lib = fq._lib.load()
    assert lib.fp4q_noalloc_scratch_bytes() == 1024
    status = torch.zeros(2, dtype=torch.int32, device=DEV)
    x = W.random_matrix(64, 512, seed=5).to(DEV)
    bad = x.clone()
    bad[3, 100] = float("inf")
    out = _empty_result(fq, 64, 512)
    fq.quantize_nvfp4_noalloc(bad, out=out, status=status)
    torch.cuda.synchronize()
    assert int(status[0].item()) & 0x1
    fq.quantize_nvfp4_noalloc(x, out=out, status=status)
    torch.cuda.synchronize()
    assert int(status[0].item()) == 0
    # a NULL status is refused before anything is enqueued
    assert lib.fp4q_quantize_nvfp4_noalloc(
        x.data_ptr(), fq._lib.F32, 64, 512, 512, None, 16, fq._lib.MSE, -3, 7, 0, 0, out.codes.data_ptr(),
        out.scales.data_ptr(), out.global_scale.data_ptr(), None, None, None, None) == fq._lib.ERR_NULL


def test_noalloc_in_a_captured_graph():
    """The call captured into a HIP graph and replayed three times, with eager
    work and synchronizations between the replays; every replay matches the
    eager workspace call on the graph's current input."""
    fq = _fq()
    rows, cols = 512, 2048
    x = W.random_matrix(rows, cols, seed=7, dist="t4", dtype=torch.bfloat16).to(DEV)
    imp = W.random_importance(cols, seed=8).to(DEV)
    out = _empty_result(fq, rows, cols)
    status = torch.zeros(2, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        fq.quantize_nvfp4_noalloc(x, imp, out=out, status=status)   # scratch address looked up eagerly
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fq.quantize_nvfp4_noalloc(x, imp, out=out, status=status)
    for k in range(3):
        x.copy_(W.random_matrix(rows, cols, seed=100 + k, dist="t4", dtype=torch.bfloat16))
        ref = fq.quantize_nvfp4(x, imp, check=True)   # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_same(out, ref)
        assert int(status[0].item()) == 0

"""Host-only checks of the Python binding's argument validation: the C ABI
sees only pointers, so the binding must refuse caller tensors whose shape,
dtype, device or layout would let the library read or write outside them.
No library call is made here."""

import pytest
import torch

import fp4_post_quantization_amd as fq

CPU = torch.device("cpu")


def _nv_result(rows, cols):
    return fq.NVFP4Result(torch.empty((rows, cols // 2), dtype=torch.uint8),
                          torch.empty((rows, cols // 16), dtype=torch.uint8),
                          torch.empty(1),
                          torch.empty((rows, cols // 16)),
                          torch.empty((rows, cols // 16), dtype=torch.int8))


def test_matching_result_passes():
    fq._check_result(_nv_result(8, 64), 8, 64, 16, CPU)
    mx = fq.MXFP4Result(torch.empty((8, 32), dtype=torch.uint8), torch.empty((8, 2), dtype=torch.uint8), None, None)
    fq._check_result(mx, 8, 64, 32, CPU)


@pytest.mark.parametrize("field,bad", [
    ("codes", torch.empty((8, 16), dtype=torch.uint8)),                  # too small
    ("scales", torch.empty((8, 4), dtype=torch.int8)),                   # wrong dtype
    ("global_scale", torch.empty(2)),                                    # wrong shape
    ("block_loss", torch.empty((8, 8))[:, ::2]),                         # strided view
    ("offsets", torch.empty((4, 4), dtype=torch.int8)),                  # wrong rows
])
def test_mismatched_result_field_is_refused(field, bad):
    out = _nv_result(8, 64)._replace(**{field: bad})
    with pytest.raises(ValueError, match=field):
        fq._check_result(out, 8, 64, 16, CPU)


def test_result_on_another_device_is_refused():
    with pytest.raises(ValueError):
        fq._check_result(_nv_result(8, 64), 8, 64, 16, torch.device("cuda", 0))


def test_given_tensor_checks():
    t = torch.empty((4, 8))
    assert fq._given(t, (4, 8), torch.float32, CPU, "t") is t
    for bad in (t.t(), t[:, :4], t.double(), torch.empty((2, 8))):
        with pytest.raises(ValueError):
            fq._given(bad, (4, 8), torch.float32, CPU, "t")
    with pytest.raises(ValueError):
        fq._given([1.0], (1,), torch.float32, CPU, "t")


def test_workspace_must_be_dense_uint8_on_the_device():
    with pytest.raises(ValueError):
        fq._ws(torch.zeros(64, dtype=torch.int32), CPU)
    with pytest.raises(ValueError):
        fq._ws(torch.zeros(128, dtype=torch.uint8)[::2], CPU)
    with pytest.raises(ValueError):
        fq._ws(torch.zeros(64, dtype=torch.uint8), torch.device("cuda", 0))
    ws = torch.zeros(64, dtype=torch.uint8)
    assert fq._ws(ws, CPU) is ws


def test_product_operands_must_share_a_gpu():
    with pytest.raises(ValueError, match="device tensors"):
        fq._same_device(CPU, b_codes=torch.empty(1))
    with pytest.raises(ValueError, match="b_codes"):
        fq._same_device(torch.device("cuda", 0), b_codes=torch.empty(1))

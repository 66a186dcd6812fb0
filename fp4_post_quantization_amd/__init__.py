"""fp4_post_quantization_amd -- FP4 microscaling block quantization with
block-scale search on AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/fp4q.h (libfp4q.so, built in
place).  It only marshals arguments: torch supplies device memory and the
current HIP stream, and every step of the computation runs in the library's
HIP kernels.  There is no CPU fallback; a missing library raises.

    quantize_nvfp4(x, importance=None, window=None, hadamard_n=0, ...)
    quantize_mxfp4(x, importance=None, window=(-1, 0), hadamard_n=0, ...)
    quantize_relaxed(x, scales, coeffs=None, fmt="nvfp4", global_scale=None, sub=8, ...)
    gptq_nvfp4(w, hinv_chol, importance=None, window=None, global_scale=None, ...)
    dequantize(fmt, codes, scales, global_scale=None)
    block_hadamard(x, n)
"""

from typing import NamedTuple, Optional

import torch

from . import _lib as L
from ._lib import FP4QError  # noqa: F401

__all__ = [
    "quantize_nvfp4", "quantize_nvfp4_noalloc", "global_scale_nvfp4", "quantize_mxfp4", "quantize_relaxed",
    "gptq_nvfp4", "gptq_mxfp4", "gptq_static_nvfp4", "gptq_static_mxfp4", "dequantize",
    "block_hadamard", "gemm_mxfp4", "gemm_nvfp4",
    "NVFP4Result", "MXFP4Result", "workspace", "read_status", "clear_status", "FP4QError",
]


class NVFP4Result(NamedTuple):
    codes: torch.Tensor         # uint8 [R, C/2] packed E2M1 codes
    scales: torch.Tensor        # uint8 [R, C/16] E4M3 block-scale patterns
    global_scale: torch.Tensor  # float32 [1]
    block_loss: Optional[torch.Tensor]  # float32 [R, C/16]
    offsets: Optional[torch.Tensor]     # int8 [R, C/16]


class MXFP4Result(NamedTuple):
    codes: torch.Tensor         # uint8 [R, C/2]
    scales: torch.Tensor        # uint8 [R, C/32] E8M0 bytes
    block_loss: Optional[torch.Tensor]  # float32 [R, C/32]
    offsets: Optional[torch.Tensor]     # int8 [R, C/32]


_WORKSPACES = {}


def workspace(device=None):
    """The workspace used when none is passed: one per device and stream,
    taken for the device's current stream (calls on one stream run in
    order, so they may share it; calls on different streams get different
    ones).  Its status word holds the data errors of the last call on it
    (every call writes it on its stream)."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    index = device.index if device.index is not None else torch.cuda.current_device()
    key = (index, _stream(device))
    ws = _WORKSPACES.get(key)
    if ws is None:
        ws = torch.zeros(L.load().fp4q_workspace_bytes(), dtype=torch.uint8, device=torch.device("cuda", index))
        _WORKSPACES[key] = ws
    return ws


def read_status(ws):
    """Device status word (FP4Q_DATA_* bits of the last call on this
    workspace) after the stream has finished."""
    return int(ws[:4].view(torch.int32).item())


def clear_status(ws):
    ws[:4].zero_()


def _check_data(ws):
    torch.cuda.current_stream(ws.device).synchronize()
    st = read_status(ws)
    if st:
        names = []
        if st & L.DATA_NONFINITE_INPUT:
            names.append("non-finite input")
        if st & L.DATA_BAD_IMPORTANCE:
            names.append("negative or non-finite importance")
        if st & L.DATA_BAD_GLOBAL_SCALE:
            names.append("invalid global scale")
        if st & L.DATA_BAD_SCALE:
            names.append("invalid scale or coefficient")
        if st & L.DATA_BAD_HESSIAN:
            names.append("invalid inverse-Hessian factor")
        if st & L.DATA_BAD_PERM:
            names.append("processing order is not a permutation")
        raise FP4QError("data error: " + ", ".join(names))


def _dtype_code(t):
    if t.dtype == torch.float32:
        return L.F32
    if t.dtype == torch.bfloat16:
        return L.BF16
    raise TypeError(f"x must be float32 or bfloat16, got {t.dtype}")


def _matrix(x):
    if x.dim() != 2:
        raise ValueError("x must be a 2-D row-major matrix")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    # rows must not overlap (a broadcast view has row stride 0): copy unless
    # the elements are unit-strided and rows sit at least one row apart
    if (x.stride(1) != 1 and x.size(1) > 1) or (x.size(0) > 1 and x.stride(0) < x.size(1)):
        x = x.contiguous()
    ld = x.stride(0) if x.size(0) > 1 else x.size(1)
    return x, max(ld, x.size(1))


# torch's raw query of the current stream handle (the one its own generated
# code uses) costs far less host time per call than building a Stream object
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    """The device's current HIP stream handle, as an int."""
    index = device.index if device.index is not None else torch.cuda.current_device()
    if _RAW_STREAM is not None:
        return int(_RAW_STREAM(index))
    return int(torch.cuda.current_stream(index).cuda_stream)


def ctypes_ptr(v):
    return None if v is None else int(v)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _importance(importance, cols, device):
    if importance is None:
        return None
    imp = torch.as_tensor(importance, dtype=torch.float32, device=device).contiguous()
    if imp.numel() != cols:
        raise ValueError("importance must have one entry per column")
    return imp


def _given(t, shape, dtype, device, name):
    """A tensor the caller passes for the library to read or write in place:
    checked against the shape, dtype and device it must have, and required
    to be dense, so no access can fall outside it."""
    if (not isinstance(t, torch.Tensor) or t.shape != shape or t.dtype != dtype or t.device != device
            or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")
    return t


def _ws(ws, device):
    """The caller's workspace (a dense uint8 tensor on the call's device) or
    the default one for the device's current stream."""
    if ws is None:
        return workspace(device)
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"ws must be a contiguous uint8 tensor on {device}")
    return ws


def _same_device(device, **tensors):
    """Every operand of a product on the device of its first operand (a GPU)."""
    if device.type != "cuda":
        raise ValueError("the operands must be device tensors")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the operands on {device}")


def _check_result(out, rows, cols, block, device):
    """A caller-given NVFP4Result / MXFP4Result, checked like _given (one
    pass of inexpensive tests; the per-field checks name a mismatch)."""
    per_block = (rows, cols // block)
    c, sc, g = out.codes, out.scales, getattr(out, "global_scale", None)
    bl, of = out.block_loss, out.offsets
    ok = (isinstance(c, torch.Tensor) and c.shape == (rows, cols // 2) and c.dtype == torch.uint8
          and c.device == device and c.is_contiguous()
          and isinstance(sc, torch.Tensor) and sc.shape == per_block and sc.dtype == torch.uint8
          and sc.device == device and sc.is_contiguous()
          and (g is None or (isinstance(g, torch.Tensor) and g.shape == (1,) and g.dtype == torch.float32
                             and g.device == device))
          and (bl is None or (isinstance(bl, torch.Tensor) and bl.shape == per_block and bl.dtype == torch.float32
                              and bl.device == device and bl.is_contiguous()))
          and (of is None or (isinstance(of, torch.Tensor) and of.shape == per_block and of.dtype == torch.int8
                              and of.device == device and of.is_contiguous())))
    if ok:
        return
    _given(c, (rows, cols // 2), torch.uint8, device, "out.codes")
    _given(sc, per_block, torch.uint8, device, "out.scales")
    if g is not None:
        _given(g, (1,), torch.float32, device, "out.global_scale")
    if bl is not None:
        _given(bl, per_block, torch.float32, device, "out.block_loss")
    if of is not None:
        _given(of, per_block, torch.int8, device, "out.offsets")


def quantize_nvfp4(x, importance=None, window=None, hadamard_n=0, global_scale=None, *,
                   out=None, with_loss=True, with_offsets=True, ws=None, check=False, accumulate_status=False):
    """NVFP4 ScaleSweep quantization of a 2-D float32/bfloat16 device tensor.

    importance: per-column weights -> WMSE (default window (-8, 7)); None ->
    MSE (default window (-3, 7)).  global_scale: a given S (float or [1]
    tensor; passing ``out.global_scale`` itself copies nothing) instead of
    max|x|/1536.  out: a preallocated NVFP4Result to write into.  check: synchronize and raise on data errors.
    accumulate_status: add this call's data errors to the workspace's status
    word instead of replacing it (FP4Q_ACCUMULATE_STATUS).
    """
    lib = L.load()
    x, ld = _matrix(x)
    rows, cols = x.shape
    dev = x.device
    imp = _importance(importance, cols, dev)
    loss = L.WMSE if imp is not None else L.MSE
    if window is None:
        window = (-8, 7) if imp is not None else (-3, 7)
    if out is None:
        out = NVFP4Result(
            codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
            scales=torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev),
            global_scale=torch.empty(1, dtype=torch.float32, device=dev),
            block_loss=torch.empty((rows, cols // 16), dtype=torch.float32, device=dev) if with_loss else None,
            offsets=torch.empty((rows, cols // 16), dtype=torch.int8, device=dev) if with_offsets else None,
        )
    else:
        _check_result(out, rows, cols, 16, dev)
    flags = 0
    if global_scale is not None:
        same = isinstance(global_scale, torch.Tensor) and global_scale.data_ptr() == out.global_scale.data_ptr()
        if not same:
            out.global_scale.copy_(torch.as_tensor(global_scale, dtype=torch.float32).reshape(1))
        flags |= L.GIVEN_SCALE
    if accumulate_status:
        flags |= L.ACCUMULATE_STATUS
    ws = _ws(ws, dev)
    L.check(lib.fp4q_quantize_nvfp4(
        x.data_ptr(), _dtype_code(x), rows, cols, ld, _ptr(imp), 16, loss, int(window[0]), int(window[1]),
        int(hadamard_n), flags, out.codes.data_ptr(), out.scales.data_ptr(), out.global_scale.data_ptr(),
        _ptr(out.block_loss), _ptr(out.offsets), ws.data_ptr(), ws.numel(), _stream(dev)))
    if check:
        _check_data(ws)
    return out


def quantize_nvfp4_noalloc(x, importance=None, window=None, hadamard_n=0, *, out, status,
                           given_scale=False, accumulate_status=False):
    """quantize_nvfp4 through fp4q_quantize_nvfp4_noalloc: no workspace and
    no device allocation in the call.  Every tensor is the caller's and is
    used in place: x a dense row-major float32/bfloat16 matrix, importance a
    dense float32 [cols] vector (WMSE) or None, out a preallocated
    NVFP4Result, status a [2] int32 device tensor (element 0 receives the
    data-error bits, element 1 the call's tag).
    given_scale: out.global_scale already holds S (FP4Q_GIVEN_SCALE)."""
    lib = L.load()
    if x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D device tensor")
    rows, cols = x.shape
    dev = x.device
    if importance is not None:
        _given(importance, (cols,), torch.float32, dev, "importance")
    loss = L.WMSE if importance is not None else L.MSE
    if window is None:
        window = (-8, 7) if importance is not None else (-3, 7)
    _check_result(out, rows, cols, 16, dev)
    if out.global_scale is None:
        raise ValueError("out.global_scale is required")
    _given(status, (2,), torch.int32, dev, "status")
    flags = (L.GIVEN_SCALE if given_scale else 0) | (L.ACCUMULATE_STATUS if accumulate_status else 0)
    L.check(lib.fp4q_quantize_nvfp4_noalloc(
        x.data_ptr(), _dtype_code(x), rows, cols, cols, _ptr(importance), 16, loss, int(window[0]),
        int(window[1]), int(hadamard_n), flags, out.codes.data_ptr(), out.scales.data_ptr(),
        out.global_scale.data_ptr(), _ptr(out.block_loss), _ptr(out.offsets), status.data_ptr(), _stream(dev)))
    return out


def global_scale_nvfp4(x, hadamard_n=0, *, out=None, ws=None):
    """The NVFP4 global scale S = max|x| / 1536 (after the optional rotation)
    as a [1] float32 device tensor, enqueued on the current stream: the first
    step of quantize_nvfp4, which takes it back through ``global_scale``."""
    lib = L.load()
    x, ld = _matrix(x)
    rows, cols = x.shape
    dev = x.device
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=dev)
    _given(out, (1,), torch.float32, dev, "out")
    ws = _ws(ws, dev)
    L.check(lib.fp4q_global_scale_nvfp4(x.data_ptr(), _dtype_code(x), rows, cols, ld, int(hadamard_n),
                                        out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    return out


def quantize_mxfp4(x, importance=None, window=(-1, 0), hadamard_n=0, *, out=None, with_loss=True,
                   with_offsets=True, ws=None, check=False):
    """MXFP4 quantization (E8M0 scales, blocks of 32) with an exponent-window
    search; window (0, 0) is the AbsMax rule."""
    lib = L.load()
    x, ld = _matrix(x)
    rows, cols = x.shape
    dev = x.device
    imp = _importance(importance, cols, dev)
    loss = L.WMSE if imp is not None else L.MSE
    if out is None:
        out = MXFP4Result(
            codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
            scales=torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev),
            block_loss=torch.empty((rows, cols // 32), dtype=torch.float32, device=dev) if with_loss else None,
            offsets=torch.empty((rows, cols // 32), dtype=torch.int8, device=dev) if with_offsets else None,
        )
    else:
        _check_result(out, rows, cols, 32, dev)
    ws = _ws(ws, dev)
    L.check(lib.fp4q_quantize_mxfp4(
        x.data_ptr(), _dtype_code(x), rows, cols, ld, _ptr(imp), 32, loss, int(window[0]), int(window[1]),
        int(hadamard_n), out.codes.data_ptr(), out.scales.data_ptr(), _ptr(out.block_loss),
        _ptr(out.offsets), ws.data_ptr(), ws.numel(), _stream(dev)))
    if check:
        _check_data(ws)
    return out


def quantize_relaxed(x, scales, coeffs=None, fmt="nvfp4", global_scale=None, sub=8, *, dequant=True,
                     out_codes=None, out_dequant=None, ws=None, check=False):
    """FOCUS forward quantizer: codes under the quantization scale
    S_dq * c_k of each sub-block (coeffs: float16 [R, C/sub] or None for all
    ones), plus the dequantized values q * S_dq when ``dequant``.
    Returns (codes, dequantized or None)."""
    lib = L.load()
    x, ld = _matrix(x)
    rows, cols = x.shape
    dev = x.device
    fmt_code = {"nvfp4": L.NVFP4, "mxfp4": L.MXFP4}[fmt]
    block = 16 if fmt_code == L.NVFP4 else 32
    scales = _given(scales.contiguous(), (rows, cols // block), torch.uint8, dev, "scales")
    c = None
    if coeffs is not None:
        c = torch.as_tensor(coeffs, device=dev).to(torch.float16).contiguous()
        if c.numel() != rows * (cols // sub):
            raise ValueError("coeffs must hold one entry per sub-block")
    gs = None
    if fmt_code == L.NVFP4:
        gs = torch.as_tensor(global_scale, dtype=torch.float32, device=dev).reshape(1)
    if out_codes is not None:
        codes = _given(out_codes, (rows, cols // 2), torch.uint8, dev, "out_codes")
    else:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    dq = None
    if dequant:
        if out_dequant is not None:
            dq = _given(out_dequant, (rows, cols), torch.float32, dev, "out_dequant")
        else:
            dq = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    ws = _ws(ws, dev)
    L.check(lib.fp4q_quantize_relaxed(
        fmt_code, x.data_ptr(), _dtype_code(x), rows, cols, ld, scales.data_ptr(), _ptr(gs), _ptr(c), int(sub),
        codes.data_ptr(), _ptr(dq), ws.data_ptr(), ws.numel(), _stream(dev)))
    if check:
        _check_data(ws)
    return codes, dq


def _gptq_operands(w):
    """The weight as the library reads it, and float32 working storage.  A
    float32 weight with unit column stride, a row stride that is a multiple
    of 4 and 16-byte alignment is read in place (the library reads each
    column from it until an update first writes the working copy); any other
    is copied into the working storage first."""
    if w.dim() != 2 or not w.is_cuda:
        raise ValueError("w must be a 2-D device tensor")
    rows, cols = w.shape
    work = torch.empty((rows, cols), dtype=torch.float32, device=w.device)
    if (w.dtype == torch.float32 and w.stride(1) == 1 and w.stride(0) % 4 == 0 and w.stride(0) >= cols
            and w.data_ptr() % 16 == 0):
        return w, w.stride(0), work
    work.copy_(w)
    return None, 0, work


def gptq_nvfp4(w, hinv_chol, importance=None, window=None, global_scale=None, *, ws=None, check=False):
    """GPTQ with ScaleSweep group scales (NVFP4).  w: [R, C] weight (any
    float dtype, C a multiple of 128; left unchanged); hinv_chol: [C, C]
    upper Cholesky factor U of the damped inverse Hessian (H^-1 = U^T U);
    importance: per-column WMSE weights or None (MSE).  Returns an
    NVFP4Result without losses and offsets."""
    lib = L.load()
    src, ld_src, work = _gptq_operands(w)
    rows, cols = w.shape
    dev = w.device
    U = torch.as_tensor(hinv_chol, dtype=torch.float32, device=dev).contiguous()
    if U.shape != (cols, cols):
        raise ValueError("hinv_chol must be [cols, cols]")
    imp = _importance(importance, cols, dev)
    if window is None:
        window = (-8, 7) if imp is not None else (-3, 7)
    out = NVFP4Result(
        codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
        scales=torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev),
        global_scale=torch.empty(1, dtype=torch.float32, device=dev),
        block_loss=None, offsets=None)
    flags = 0
    if global_scale is not None:
        out.global_scale.copy_(torch.as_tensor(global_scale, dtype=torch.float32).reshape(1))
        flags |= L.GIVEN_SCALE
    ws = _ws(ws, dev)
    L.check(lib.fp4q_gptq_nvfp4(
        work.data_ptr(), rows, cols, work.stride(0), _ptr(src), ld_src, U.data_ptr(), _ptr(imp),
        int(window[0]), int(window[1]), flags, out.codes.data_ptr(), out.scales.data_ptr(),
        out.global_scale.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    if check:
        _check_data(ws)
    return out


def gptq_mxfp4(w, hinv_chol, importance=None, window=(-1, 0), *, ws=None, check=False):
    """GPTQ with MXFP4 group scales.  w: [R, C] weight (C a multiple of
    128; left unchanged); hinv_chol: [C, C] upper Cholesky factor U of the
    damped inverse Hessian; importance: per-column WMSE weights or None
    (MSE); window: E8M0 exponent offsets around each group's base exponent.
    Returns an MXFP4Result without losses and offsets."""
    lib = L.load()
    src, ld_src, work = _gptq_operands(w)
    rows, cols = w.shape
    dev = w.device
    U = torch.as_tensor(hinv_chol, dtype=torch.float32, device=dev).contiguous()
    if U.shape != (cols, cols):
        raise ValueError("hinv_chol must be [cols, cols]")
    imp = _importance(importance, cols, dev)
    out = MXFP4Result(
        codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
        scales=torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev),
        block_loss=None, offsets=None)
    ws = _ws(ws, dev)
    L.check(lib.fp4q_gptq_mxfp4(
        work.data_ptr(), rows, cols, work.stride(0), _ptr(src), ld_src, U.data_ptr(), _ptr(imp),
        int(window[0]), int(window[1]), out.codes.data_ptr(), out.scales.data_ptr(), ws.data_ptr(), ws.numel(),
        _stream(dev)))
    if check:
        _check_data(ws)
    return out


def _gptq_static_operands(w, perm, hinv_chol, importance):
    """Static-order GPTQ operands: the weight as a float32 source the
    library can read (copied when it is not one), float32 working storage,
    the order as a dense int32 device vector, U and the importance (16-byte
    aligned) and a workspace of the size the call needs."""
    if w.dim() != 2 or not w.is_cuda:
        raise ValueError("w must be a 2-D device tensor")
    rows, cols = w.shape
    dev = w.device
    src = w
    if not (w.dtype == torch.float32 and w.stride(1) == 1 and w.stride(0) % 4 == 0 and w.stride(0) >= cols
            and w.data_ptr() % 16 == 0):
        src = w.to(torch.float32).contiguous()
    work = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    p = torch.as_tensor(perm, device=dev).to(torch.int32).contiguous()
    if p.shape != (cols,):
        raise ValueError("perm must have one entry per column")
    U = torch.as_tensor(hinv_chol, dtype=torch.float32, device=dev).contiguous()
    if U.shape != (cols, cols):
        raise ValueError("hinv_chol must be [cols, cols]")
    imp = _importance(importance, cols, dev)
    if imp is not None and imp.data_ptr() % 16:
        imp = imp.clone()
    lib = L.load()
    ws = torch.empty(lib.fp4q_gptq_static_workspace_bytes(rows, cols) + 256, dtype=torch.uint8, device=dev)
    off = (-ws.data_ptr()) % 256
    return src, work, p, U, imp, ws[off:off + lib.fp4q_gptq_static_workspace_bytes(rows, cols)]


def gptq_static_nvfp4(w, perm, hinv_chol, importance=None, window=None, global_scale=None, *, check=False):
    """GPTQ with static activation reordering, NVFP4 group scales.  w: [R, C]
    weight in the stored order (C a multiple of 128; left unchanged); perm:
    [C] processing order (slot j takes stored column perm[j]); hinv_chol:
    [C, C] upper Cholesky factor of the damped inverse Hessian permuted to
    that order; importance: stored-order WMSE weights or None.  Every
    group's scale is the sweep's on w as given.  Returns an NVFP4Result (codes
    and scales in the stored order) without losses and offsets."""
    lib = L.load()
    src, work, p, U, imp, ws = _gptq_static_operands(w, perm, hinv_chol, importance)
    rows, cols = w.shape
    dev = w.device
    if window is None:
        window = (-8, 7) if imp is not None else (-3, 7)
    out = NVFP4Result(
        codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
        scales=torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev),
        global_scale=torch.empty(1, dtype=torch.float32, device=dev),
        block_loss=None, offsets=None)
    flags = 0
    if global_scale is not None:
        out.global_scale.copy_(torch.as_tensor(global_scale, dtype=torch.float32).reshape(1))
        flags |= L.GIVEN_SCALE
    L.check(lib.fp4q_gptq_static_nvfp4(
        work.data_ptr(), rows, cols, work.stride(0), src.data_ptr(), src.stride(0), p.data_ptr(), U.data_ptr(),
        _ptr(imp), int(window[0]), int(window[1]), flags, out.codes.data_ptr(), out.scales.data_ptr(),
        out.global_scale.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    if check:
        _check_data(ws)
    return out


def gptq_static_mxfp4(w, perm, hinv_chol, importance=None, window=(-1, 0), *, check=False):
    """gptq_static_nvfp4 with MXFP4 group exponents (the exponent sweep's on
    w as given, window of exponent offsets).  Returns an MXFP4Result (codes
    and E8M0 bytes in the stored order) without losses and offsets."""
    lib = L.load()
    src, work, p, U, imp, ws = _gptq_static_operands(w, perm, hinv_chol, importance)
    rows, cols = w.shape
    dev = w.device
    out = MXFP4Result(
        codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
        scales=torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev),
        block_loss=None, offsets=None)
    L.check(lib.fp4q_gptq_static_mxfp4(
        work.data_ptr(), rows, cols, work.stride(0), src.data_ptr(), src.stride(0), p.data_ptr(), U.data_ptr(),
        _ptr(imp), int(window[0]), int(window[1]), out.codes.data_ptr(), out.scales.data_ptr(), ws.data_ptr(),
        ws.numel(), _stream(dev)))
    if check:
        _check_data(ws)
    return out


def dequantize(fmt, codes, scales, global_scale=None, out=None):
    """Decode packed codes and block scales to float32 ([R, C])."""
    lib = L.load()
    fmt_code = {"nvfp4": L.NVFP4, "mxfp4": L.MXFP4}[fmt]
    block = 16 if fmt_code == L.NVFP4 else 32
    rows, half = codes.shape
    cols = half * 2
    dev = codes.device
    codes = _given(codes.contiguous(), (rows, half), torch.uint8, dev, "codes")
    scales = _given(scales.contiguous(), (rows, cols // block), torch.uint8, dev, "scales")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    _given(out, (rows, cols), torch.float32, dev, "out")
    gs = None
    if fmt_code == L.NVFP4:
        gs = torch.as_tensor(global_scale, dtype=torch.float32, device=dev).reshape(1)
    L.check(lib.fp4q_dequantize(fmt_code, codes.data_ptr(), scales.data_ptr(), _ptr(gs), rows, cols, block,
                                out.data_ptr(), _stream(dev)))
    return out


def block_hadamard(x, n, out=None):
    """Rotate each row's n-column groups by H_n / sqrt(n) (float32 output)."""
    lib = L.load()
    x, ld = _matrix(x)
    rows, cols = x.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=x.device)
    _given(out, (rows, cols), torch.float32, x.device, "out")
    L.check(lib.fp4q_block_hadamard(x.data_ptr(), _dtype_code(x), rows, cols, ld, int(n), out.data_ptr(),
                                    _stream(x.device)))
    return out


def gemm_mxfp4(a, b, *, alpha=1.0, out_dtype=torch.float32, out=None, workspace_buf=None, use_workspace=True):
    """C = alpha * A_hat @ B_hat^T for MXFP4 operands (W4A4).

    ``a`` and ``b`` are MXFP4Result (or (codes, scales) pairs) as written by
    ``quantize_mxfp4``: A is M x K (activations), B is N x K (weights).
    Returns C [M, N] in float32 or bfloat16.  Few-token products (M <= 16,
    or M <= 64 on N <= 4096; K a multiple of 512, at most 16384, or 8192
    above 16 tokens) run in one kernel without a workspace.  Otherwise, with ``use_workspace`` (and K a multiple of
    256), the library gets the workspace that
    ``fp4q_gemm_mxfp4_workspace_bytes`` asks for (``workspace_buf`` or a
    fresh one): large products copy the scales stage-major into it (same
    result), other products of up to 64 tokens split K and keep their
    partial sums there (added in K order: the result can differ in
    rounding)."""
    lib = L.load()
    ac, as_ = (a.codes, a.scales) if isinstance(a, MXFP4Result) else a
    bc, bs = (b.codes, b.scales) if isinstance(b, MXFP4Result) else b
    m, kh = ac.shape
    n, kh2 = bc.shape
    if kh != kh2:
        raise ValueError(f"K mismatch: A has {2 * kh}, B has {2 * kh2}")
    k = 2 * kh
    dev = ac.device
    ac, as_, bc, bs = (t.contiguous() for t in (ac, as_, bc, bs))
    _same_device(dev, a_scales=as_, b_codes=bc, b_scales=bs, out=out, workspace_buf=workspace_buf)
    if as_.shape != (m, k // 32) or bs.shape != (n, k // 32):
        raise ValueError("scales must be rows x K/32")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    if (out.dtype not in (torch.float32, torch.bfloat16) or out.shape != (m, n) or out.stride(1) != 1
            or (m > 1 and out.stride(0) < n)):
        raise ValueError("out must be a row-major float32 or bfloat16 [M, N] tensor")
    code = L.F32 if out.dtype == torch.float32 else L.BF16
    need = lib.fp4q_gemm_mxfp4_workspace_bytes(m, n, k) if use_workspace else 0
    if workspace_buf is not None and not workspace_buf.is_contiguous():
        raise ValueError("workspace_buf must be contiguous")
    if need and (workspace_buf is None or workspace_buf.numel() < need):
        workspace_buf = torch.empty(need, dtype=torch.uint8, device=dev)
    L.check(lib.fp4q_gemm_mxfp4(ac.data_ptr(), as_.data_ptr(), bc.data_ptr(), bs.data_ptr(), m, n, k,
                                float(alpha), code, out.data_ptr(), out.stride(0) if m > 1 else n,
                                _ptr(workspace_buf) if need else None, workspace_buf.numel() if need else 0,
                                _stream(dev)))
    return out


def gemm_nvfp4(a, b, *, out_dtype=torch.float32, out=None, workspace_buf=None):
    """C = fp32(S_a S_b) * A_hat @ B_hat^T for NVFP4 operands (NVFP4Result
    or (codes, scales, global_scale) triples as written by quantize_nvfp4):
    A is M x K, B is N x K.  Large products decode the operands to bfloat16
    (exact) in a workspace, allocated here unless ``workspace_buf`` is given;
    smaller ones decode in registers.  Few-token products (M <= 32, or
    M <= 64 on N <= 4096; K a multiple of 256) need a workspace only when
    they split K, for the partial sums.  ``fp4q_gemm_nvfp4_workspace_bytes``
    gives the size in every case."""
    lib = L.load()
    ac, as_, ag = (a.codes, a.scales, a.global_scale) if isinstance(a, NVFP4Result) else a
    bc, bs, bg = (b.codes, b.scales, b.global_scale) if isinstance(b, NVFP4Result) else b
    m, kh = ac.shape
    n, kh2 = bc.shape
    if kh != kh2:
        raise ValueError(f"K mismatch: A has {2 * kh}, B has {2 * kh2}")
    k = 2 * kh
    dev = ac.device
    ac, as_, bc, bs = (t.contiguous() for t in (ac, as_, bc, bs))
    _same_device(dev, a_scales=as_, b_codes=bc, b_scales=bs, out=out, workspace_buf=workspace_buf)
    ag = torch.as_tensor(ag, dtype=torch.float32, device=dev).reshape(1)
    bg = torch.as_tensor(bg, dtype=torch.float32, device=dev).reshape(1)
    if as_.shape != (m, k // 16) or bs.shape != (n, k // 16):
        raise ValueError("scales must be rows x K/16")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    if (out.dtype not in (torch.float32, torch.bfloat16) or out.shape != (m, n) or out.stride(1) != 1
            or (m > 1 and out.stride(0) < n)):
        raise ValueError("out must be a row-major float32 or bfloat16 [M, N] tensor")
    need = lib.fp4q_gemm_nvfp4_workspace_bytes(m, n, k)
    if workspace_buf is not None and not workspace_buf.is_contiguous():
        raise ValueError("workspace_buf must be contiguous")
    if need and (workspace_buf is None or workspace_buf.numel() < need):
        workspace_buf = torch.empty(need, dtype=torch.uint8, device=dev)
    code = L.F32 if out.dtype == torch.float32 else L.BF16
    L.check(lib.fp4q_gemm_nvfp4(ac.data_ptr(), as_.data_ptr(), ag.data_ptr(), bc.data_ptr(), bs.data_ptr(),
                                bg.data_ptr(), m, n, k, code, out.data_ptr(), out.stride(0) if m > 1 else n,
                                _ptr(workspace_buf) if need else None, workspace_buf.numel() if need else 0,
                                _stream(dev)))
    return out

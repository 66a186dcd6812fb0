"""ctypes declarations of the fp4q C ABI (include/fp4q.h, include/fp4q_gemm.h)."""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; FP4Q_LIBRARY names another build of the same sources (e.g. the host-sanitized
# checking build of build.py --host-sanitize)
LIB_PATH = os.environ.get("FP4Q_LIBRARY") or os.path.join(_PKG, "libfp4q.so")

# status codes
OK, ERR_NULL, ERR_SHAPE, ERR_ARG, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = range(7)
# enums
F32, BF16 = 0, 1
MSE, WMSE = 0, 1
NVFP4, MXFP4 = 0, 1
GIVEN_SCALE = 0x1
ACCUMULATE_STATUS = 0x2
DATA_NONFINITE_INPUT = 0x1
DATA_BAD_IMPORTANCE = 0x2
DATA_BAD_GLOBAL_SCALE = 0x4
DATA_BAD_SCALE = 0x8
DATA_BAD_HESSIAN = 0x10
DATA_BAD_PERM = 0x20

EXPORTS = (
    "fp4q_version",
    "fp4q_status_string",
    "fp4q_workspace_bytes",
    "fp4q_quantize_nvfp4",
    "fp4q_quantize_nvfp4_noalloc",
    "fp4q_noalloc_scratch_bytes",
    "fp4q_global_scale_nvfp4",
    "fp4q_quantize_mxfp4",
    "fp4q_quantize_relaxed",
    "fp4q_gptq_nvfp4",
    "fp4q_gptq_mxfp4",
    "fp4q_gptq_static_workspace_bytes",
    "fp4q_gptq_static_nvfp4",
    "fp4q_gptq_static_mxfp4",
    "fp4q_dequantize",
    "fp4q_block_hadamard",
    "fp4q_gemm_mxfp4",
    "fp4q_gemm_mxfp4_workspace_bytes",
    "fp4q_gemm_nvfp4_workspace_bytes",
    "fp4q_gemm_nvfp4",
)

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "fp4q_version": (_I, []),
    "fp4q_status_string": (ctypes.c_char_p, [_I]),
    "fp4q_workspace_bytes": (_SZ, []),
    "fp4q_global_scale_nvfp4": (_I, [_P, _I, _I64, _I64, _I64, _I, _P, _P, _SZ, _P]),
    "fp4q_quantize_nvfp4": (_I, [_P, _I, _I64, _I64, _I64, _P, _I, _I, _I, _I, _I, _U32,
                                 _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fp4q_quantize_nvfp4_noalloc": (_I, [_P, _I, _I64, _I64, _I64, _P, _I, _I, _I, _I, _I, _U32,
                                         _P, _P, _P, _P, _P, _P, _P]),
    "fp4q_noalloc_scratch_bytes": (_SZ, []),
    "fp4q_quantize_mxfp4": (_I, [_P, _I, _I64, _I64, _I64, _P, _I, _I, _I, _I, _I,
                                 _P, _P, _P, _P, _P, _SZ, _P]),
    "fp4q_quantize_relaxed": (_I, [_I, _P, _I, _I64, _I64, _I64, _P, _P, _P, _I, _P, _P, _P, _SZ, _P]),
    "fp4q_gptq_nvfp4": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _P, _I, _I, _U32, _P, _P, _P, _P, _SZ, _P]),
    "fp4q_gptq_mxfp4": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _P, _I, _I, _P, _P, _P, _SZ, _P]),
    "fp4q_gptq_static_workspace_bytes": (_SZ, [_I64, _I64]),
    "fp4q_gptq_static_nvfp4": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _P, _P, _I, _I, _U32, _P, _P, _P, _P, _SZ,
                                    _P]),
    "fp4q_gptq_static_mxfp4": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _P, _P, _I, _I, _P, _P, _P, _SZ, _P]),
    "fp4q_dequantize": (_I, [_I, _P, _P, _P, _I64, _I64, _I, _P, _P]),
    "fp4q_block_hadamard": (_I, [_P, _I, _I64, _I64, _I64, _I, _P, _P]),
    "fp4q_gemm_mxfp4": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_float, _I, _P, _I64, _P, _SZ, _P]),
    "fp4q_gemm_mxfp4_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4q_gemm_nvfp4_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "fp4q_gemm_nvfp4": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _I64, _P, _SZ, _P]),
}

_lib = None


class FP4QError(RuntimeError):
    pass


def load(path=LIB_PATH):
    """Load libfp4q.so (built in-tree by ``__graft_entry__.build()`` or
    ``python -m fp4_post_quantization_amd.build``).  Raises if it is missing:
    there is no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FP4QError(f"{path} is not built; run fp4_post_quantization_amd/build.py")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status):
    if status != OK:
        msg = load().fp4q_status_string(status).decode()
        raise FP4QError(f"fp4q error {status}: {msg}")

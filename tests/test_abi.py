"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments synchronously, before anything is
enqueued on a device (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", "fp4q.h"), os.path.join(ROOT, "include", "fp4q_gemm.h")]


def _lib():
    from fp4_post_quantization_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libfp4q.so not built (run __graft_entry__.build())")
    return L, L.load()


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(fp4q_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("fp4q_quantize_nvfp4", "fp4q_quantize_mxfp4", "fp4q_dequantize", "fp4q_block_hadamard",
              "fp4q_gemm_mxfp4", "fp4q_gemm_nvfp4"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L, lib = _lib()
    names = _declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_helpers_without_gpu():
    L, lib = _lib()
    assert lib.fp4q_version() >= 100
    assert lib.fp4q_workspace_bytes() >= 256
    for code in range(7):
        assert lib.fp4q_status_string(code)
    assert lib.fp4q_status_string(0) == b"ok"


# fake, aligned device addresses: validation must reject before any use
X = 0x10000
OUT = 0x20000
WS = 0x40000


def _nv(lib, L, **kw):
    a = dict(x=X, dtype=L.BF16, rows=4, cols=64, ld=64, imp=None, block=16, loss=L.MSE, lo=-3, hi=7,
             had=0, flags=0, codes=OUT, scales=OUT, gs=OUT, bl=None, offs=None, ws=WS,
             wsb=lib.fp4q_workspace_bytes(), stream=None)
    a.update(kw)
    return lib.fp4q_quantize_nvfp4(a["x"], a["dtype"], a["rows"], a["cols"], a["ld"], a["imp"], a["block"],
                                   a["loss"], a["lo"], a["hi"], a["had"], a["flags"], a["codes"], a["scales"],
                                   a["gs"], a["bl"], a["offs"], a["ws"], a["wsb"], a["stream"])


def test_nvfp4_argument_validation():
    L, lib = _lib()
    assert _nv(lib, L, x=None) == L.ERR_NULL
    assert _nv(lib, L, codes=None) == L.ERR_NULL
    assert _nv(lib, L, gs=None) == L.ERR_NULL
    assert _nv(lib, L, loss=L.WMSE, imp=None) == L.ERR_NULL
    assert _nv(lib, L, ws=None) == L.ERR_WORKSPACE
    assert _nv(lib, L, wsb=16) == L.ERR_WORKSPACE
    assert _nv(lib, L, dtype=7) == L.ERR_ARG
    assert _nv(lib, L, loss=5) == L.ERR_ARG
    assert _nv(lib, L, lo=1) == L.ERR_ARG
    assert _nv(lib, L, hi=-1) == L.ERR_ARG
    assert _nv(lib, L, lo=-127) == L.ERR_ARG
    assert _nv(lib, L, hi=127) == L.ERR_ARG
    assert _nv(lib, L, had=8) == L.ERR_ARG
    assert _nv(lib, L, flags=0x8) == L.ERR_ARG
    assert _nv(lib, L, block=32) == L.ERR_SHAPE
    assert _nv(lib, L, cols=40, ld=40) == L.ERR_SHAPE
    assert _nv(lib, L, ld=32) == L.ERR_SHAPE
    assert _nv(lib, L, rows=-1) == L.ERR_SHAPE
    assert _nv(lib, L, cols=48, ld=48, had=32) == L.ERR_SHAPE
    assert _nv(lib, L, rows=1 << 31, cols=16, ld=16) == L.ERR_SHAPE
    assert _nv(lib, L, x=X + 2) == L.ERR_ALIGN
    assert _nv(lib, L, ld=68) == L.ERR_ALIGN            # 136-byte bf16 rows
    assert _nv(lib, L, codes=OUT + 4) == L.ERR_ALIGN
    assert _nv(lib, L, loss=L.WMSE, imp=OUT + 4) == L.ERR_ALIGN


def test_mxfp4_dequant_hadamard_validation():
    L, lib = _lib()
    wsb = lib.fp4q_workspace_bytes()
    mx = lambda **kw: lib.fp4q_quantize_mxfp4(
        kw.get("x", X), kw.get("dtype", L.F32), kw.get("rows", 2), kw.get("cols", 64), kw.get("ld", 64),
        kw.get("imp", None), kw.get("block", 32), kw.get("loss", L.MSE), kw.get("lo", -1), kw.get("hi", 0),
        kw.get("had", 0), OUT, OUT, None, None, kw.get("ws", WS), wsb, None)
    assert mx(x=None) == L.ERR_NULL
    assert mx(block=16) == L.ERR_SHAPE
    assert mx(cols=48, ld=48) == L.ERR_SHAPE
    assert mx(lo=-17) == L.ERR_ARG
    assert mx(hi=17) == L.ERR_ARG
    assert mx(ws=None) == L.ERR_WORKSPACE
    assert mx(loss=L.WMSE) == L.ERR_NULL
    dq = lambda **kw: lib.fp4q_dequantize(kw.get("fmt", L.NVFP4), kw.get("codes", OUT), OUT,
                                          kw.get("gs", OUT), 2, kw.get("cols", 64), kw.get("block", 16),
                                          kw.get("out", OUT), None)
    assert dq(fmt=9) == L.ERR_ARG
    assert dq(codes=None) == L.ERR_NULL
    assert dq(gs=None) == L.ERR_NULL
    assert dq(block=32) == L.ERR_SHAPE
    assert dq(cols=40) == L.ERR_SHAPE
    assert dq(out=OUT + 4) == L.ERR_ALIGN
    hd = lambda **kw: lib.fp4q_block_hadamard(kw.get("x", X), L.F32, 2, kw.get("cols", 64), 64,
                                              kw.get("n", 16), kw.get("out", OUT), None)
    assert hd(x=None) == L.ERR_NULL
    assert hd(n=0) == L.ERR_ARG
    assert hd(n=24) == L.ERR_ARG
    assert hd(n=128) == L.ERR_SHAPE
    assert hd(cols=40) == L.ERR_SHAPE


def test_relaxed_validation():
    L, lib = _lib()
    wsb = lib.fp4q_workspace_bytes()
    rq = lambda **kw: lib.fp4q_quantize_relaxed(
        kw.get("fmt", L.NVFP4), kw.get("x", X), L.BF16, 2, kw.get("cols", 64), kw.get("ld", 64),
        kw.get("scales", OUT), kw.get("gs", OUT), None, kw.get("sub", 8), kw.get("codes", OUT),
        kw.get("dq", None), kw.get("ws", WS), wsb, None)
    assert rq(fmt=7) == L.ERR_ARG
    assert rq(x=None) == L.ERR_NULL
    assert rq(scales=None) == L.ERR_NULL
    assert rq(gs=None) == L.ERR_NULL
    assert rq(ws=None) == L.ERR_WORKSPACE
    assert rq(sub=32) == L.ERR_ARG          # NVFP4 blocks hold 16
    assert rq(sub=3) == L.ERR_ARG
    assert rq(fmt=L.MXFP4, cols=48, ld=48) == L.ERR_SHAPE
    assert rq(ld=60) == L.ERR_SHAPE
    assert rq(codes=OUT + 4) == L.ERR_ALIGN
    assert rq(dq=OUT + 4) == L.ERR_ALIGN


def test_gptq_validation():
    L, lib = _lib()
    wsb = lib.fp4q_workspace_bytes()
    gq = lambda **kw: lib.fp4q_gptq_nvfp4(
        kw.get("w", X), 4, kw.get("cols", 128), kw.get("ld", 128), kw.get("src", None), kw.get("lds", 0),
        kw.get("u", OUT), None, kw.get("lo", -3), kw.get("hi", 7), kw.get("flags", 0), OUT, OUT,
        kw.get("gs", OUT), kw.get("ws", WS), wsb, None)
    assert gq(w=None) == L.ERR_NULL
    assert gq(u=None) == L.ERR_NULL
    assert gq(gs=None) == L.ERR_NULL
    assert gq(ws=None) == L.ERR_WORKSPACE
    assert gq(lo=-9, hi=7) == L.ERR_ARG
    assert gq(flags=4) == L.ERR_ARG
    assert gq(cols=144, ld=144) == L.ERR_SHAPE
    assert gq(ld=100) == L.ERR_SHAPE
    assert gq(ld=130) == L.ERR_ALIGN
    assert gq(u=OUT + 4) == L.ERR_ALIGN
    # a separate read-only weight: its row stride at least cols, a multiple of 4, 16-byte aligned
    assert gq(src=X, lds=100) == L.ERR_SHAPE
    assert gq(src=X, lds=130) == L.ERR_ALIGN
    assert gq(src=X + 4, lds=128) == L.ERR_ALIGN
    gm = lambda **kw: lib.fp4q_gptq_mxfp4(
        kw.get("w", X), kw.get("rows", 4), kw.get("cols", 128), kw.get("ld", 128), kw.get("src", None),
        kw.get("lds", 0), kw.get("u", OUT), None, kw.get("lo", -1), kw.get("hi", 0), OUT, OUT, kw.get("ws", WS),
        wsb, None)
    assert gm(w=None) == L.ERR_NULL
    assert gm(u=None) == L.ERR_NULL
    assert gm(ws=None) == L.ERR_WORKSPACE
    assert gm(lo=1, hi=2) == L.ERR_ARG
    assert gm(lo=-16, hi=0) == L.ERR_ARG
    assert gm(cols=160, ld=160) == L.ERR_SHAPE
    assert gm(ld=100) == L.ERR_SHAPE
    assert gm(ld=130) == L.ERR_ALIGN
    assert gm(src=X, lds=64) == L.ERR_SHAPE
    assert gm(src=X + 8, lds=128) == L.ERR_ALIGN
    # empty: the arguments pass; the call still enqueues the kernel that writes the status word,
    # whose launch needs a GPU
    assert gm(rows=0) in (L.OK, L.ERR_HIP)


def test_gptq_static_validation():
    """Static-order GPTQ: argument errors are returned before anything is
    enqueued (no GPU needed), and the workspace query covers the inverse
    order and the processing-order codes."""
    L, lib = _lib()
    assert lib.fp4q_gptq_static_workspace_bytes(4, 128) >= lib.fp4q_workspace_bytes() + 4 * 128 + 4 * 64
    assert lib.fp4q_gptq_static_workspace_bytes(-1, 128) == 0
    wsb = lib.fp4q_gptq_static_workspace_bytes(4, 128)
    big = 1 << 40
    gs = lambda **kw: lib.fp4q_gptq_static_nvfp4(
        kw.get("w", X), 4, kw.get("cols", 128), kw.get("ld", 128), kw.get("src", 0x80000), kw.get("lds", 128),
        kw.get("perm", X), kw.get("u", OUT), kw.get("imp", None), kw.get("lo", -3), kw.get("hi", 7),
        kw.get("flags", 0), kw.get("codes", OUT), OUT, kw.get("gs", OUT), kw.get("ws", WS), kw.get("wsb", big), None)
    assert gs(src=None) == L.ERR_NULL
    assert gs(perm=None) == L.ERR_NULL
    assert gs(gs=None) == L.ERR_NULL
    assert gs(ws=None) == L.ERR_WORKSPACE
    assert gs(wsb=wsb - 1) == L.ERR_WORKSPACE
    assert gs(ws=WS + 16) == L.ERR_WORKSPACE
    assert gs(lo=-9, hi=7) == L.ERR_ARG
    assert gs(flags=2) == L.ERR_ARG
    assert gs(cols=144, ld=144, lds=144) == L.ERR_SHAPE
    assert gs(cols=-128) == L.ERR_SHAPE
    assert gs(lds=100) == L.ERR_SHAPE
    assert gs(src=0x80004) == L.ERR_ALIGN
    assert gs(perm=X + 2) == L.ERR_ALIGN
    assert gs(codes=OUT + 4) == L.ERR_ALIGN
    assert gs(imp=OUT + 4) == L.ERR_ALIGN
    # the weight and the working storage must not share memory
    assert gs(src=X + 16 * 64) == L.ERR_ARG
    assert gs(src=X) == L.ERR_ARG
    gm = lambda **kw: lib.fp4q_gptq_static_mxfp4(
        X, kw.get("rows", 4), 128, 128, 0x80000, 128, kw.get("perm", X), OUT, None, kw.get("lo", -1), kw.get("hi", 0),
        OUT, OUT, WS, big, None)
    assert gm(perm=None) == L.ERR_NULL
    assert gm(lo=-17, hi=-2) == L.ERR_ARG
    assert gm(lo=0, hi=17) == L.ERR_ARG
    assert gm(rows=0) in (L.OK, L.ERR_HIP)


def test_gemm_validation():
    L, lib = _lib()

    def gm(**kw):
        return lib.fp4q_gemm_mxfp4(kw.get("a", X), kw.get("as_", OUT), kw.get("b", X), kw.get("bs", OUT),
                                   kw.get("m", 64), kw.get("n", 64), kw.get("k", 128), 1.0,
                                   kw.get("dt", L.F32), kw.get("c", WS), kw.get("ldc", 64), kw.get("ws", None),
                                   kw.get("wsb", 0), None)
    assert lib.fp4q_gemm_mxfp4_workspace_bytes(64, 32, 512) == 96 * 16 + 32
    assert lib.fp4q_gemm_mxfp4_workspace_bytes(64, 32, 384) == 0
    # few tokens: K split in 4 (16 stages of 256, at least 4 per split), partial sums 4 x 16 x 4096 floats
    assert lib.fp4q_gemm_mxfp4_workspace_bytes(16, 4096, 4096) == 4 * 16 * 4096 * 4
    assert gm(k=512, ws=WS, wsb=100) == L.ERR_WORKSPACE
    assert gm(k=512, ws=WS + 4, wsb=1 << 20) == L.ERR_ALIGN
    assert gm(a=None) == L.ERR_NULL
    assert gm(bs=None) == L.ERR_NULL
    assert gm(c=None) == L.ERR_NULL
    assert gm(dt=7) == L.ERR_ARG
    assert gm(k=48) == L.ERR_SHAPE
    assert gm(k=0) == L.ERR_SHAPE
    assert gm(m=-1) == L.ERR_SHAPE
    assert gm(ldc=63) == L.ERR_SHAPE
    assert gm(a=X + 8) == L.ERR_ALIGN
    assert gm(c=WS + 2) == L.ERR_ALIGN
    # empty products need no pointers and enqueue nothing
    assert gm(m=0, a=None, as_=None, c=None) == L.OK
    assert gm(n=0, b=None, bs=None, c=None) == L.OK


def test_global_scale_nvfp4_validation():
    L, lib = _lib()

    def gs(**kw):
        return lib.fp4q_global_scale_nvfp4(kw.get("x", X), kw.get("dt", L.BF16), kw.get("rows", 64),
                                           kw.get("cols", 256), kw.get("ld", 256), kw.get("had", 0),
                                           kw.get("g", OUT), kw.get("ws", WS), kw.get("wsb", 1 << 20), None)
    assert gs(g=None) == L.ERR_NULL
    assert gs(x=None) == L.ERR_NULL
    assert gs(ws=None) == L.ERR_WORKSPACE
    assert gs(wsb=16) == L.ERR_WORKSPACE
    assert gs(dt=7) == L.ERR_ARG
    assert gs(had=8) == L.ERR_ARG
    assert gs(cols=40, ld=40) == L.ERR_SHAPE
    assert gs(had=32, cols=48, ld=48) == L.ERR_SHAPE
    assert gs(ld=100) == L.ERR_SHAPE
    assert gs(x=X + 4) == L.ERR_ALIGN


def test_gemm_nvfp4_validation():
    L, lib = _lib()
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(64, 32, 48) == (64 + 32) * 64 * 2
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(64, 32, 0) == 0
    # products of at most 16 tokens with K a multiple of 256 (up to 16384) decode in registers
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(16, 4096, 4096) == 0
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(1, 4096, 16384) == 0
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(17, 4096, 4096) == 0  # up to 64 tokens on 4096 columns
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(17, 8192, 4096) == 0  # up to 32 tokens on any width
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(33, 8192, 4096) == (33 + 8192) * 4096 * 2
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(65, 1024, 4096) == (65 + 1024) * 4096 * 2
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(16, 4096, 4224) == (16 + 4096) * 4224 * 2
    # K split over two workgroups per column tile: room for their partial sums
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(16, 64, 32768) == 2 * 16 * 64 * 4
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(20, 4096, 14336) == 2 * 20 * 4096 * 4
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(60, 2048, 14336) == 4 * 60 * 2048 * 4
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(16, 64, 65536) == 4 * 16 * 64 * 4
    assert lib.fp4q_gemm_nvfp4_workspace_bytes(16, 64, 131072) == (16 + 64) * 131072 * 2

    def gn(**kw):
        m, n, k = kw.get("m", 64), kw.get("n", 64), kw.get("k", 128)
        return lib.fp4q_gemm_nvfp4(kw.get("a", X), kw.get("as_", OUT), kw.get("ag", OUT), X, OUT, OUT, m, n, k,
                                   kw.get("dt", L.F32), kw.get("c", WS), kw.get("ldc", 64), kw.get("ws", WS),
                                   kw.get("wsb", 1 << 30), None)
    assert gn(a=None) == L.ERR_NULL
    assert gn(ag=None) == L.ERR_NULL
    assert gn(dt=5) == L.ERR_ARG
    assert gn(k=40) == L.ERR_SHAPE
    assert gn(ldc=10) == L.ERR_SHAPE
    assert gn(ws=None) == L.ERR_WORKSPACE
    assert gn(wsb=100) == L.ERR_WORKSPACE
    assert gn(ws=WS + 8) == L.ERR_ALIGN
    assert gn(ag=OUT + 2) == L.ERR_ALIGN
    assert gn(m=0, a=None, ag=None, c=None, ws=None) == L.OK
    # the few-token path needs 16-byte aligned codes and scales, and no workspace
    assert gn(m=4, k=512, as_=OUT + 4, ws=None) == L.ERR_ALIGN
    assert gn(m=4, k=512, a=X + 8, ws=None) == L.ERR_ALIGN


def test_empty_shapes_need_no_device_for_dequant_and_hadamard():
    L, lib = _lib()
    assert lib.fp4q_dequantize(L.NVFP4, OUT, OUT, OUT, 0, 64, 16, OUT, None) == L.OK
    assert lib.fp4q_block_hadamard(X, L.F32, 0, 64, 64, 16, OUT, None) == L.OK


def test_binding_raises_without_library(tmp_path):
    from fp4_post_quantization_amd import _lib as L
    saved = L._lib
    L._lib = None
    try:
        with pytest.raises(L.FP4QError):
            L.load(str(tmp_path / "missing.so"))
    finally:
        L._lib = saved

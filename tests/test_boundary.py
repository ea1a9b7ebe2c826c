"""C-ABI boundary tests that need no GPU.

The library is loaded and every symbol declared in include/gated_rmsnorm.h is
looked up.  Then each argument rule is exercised with calls that the library
must reject before enqueuing anything (fake, never-dereferenced pointers):
no call here reaches the GPU.
"""
import math
import pathlib
import re

import pytest
import torch

from silu_gated_rmsnorm_amd import binding

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "gated_rmsnorm.h"

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, WORKSPACE, EPS, HIP, ARG, SCRATCH = range(11)
ROWS = 10
ACT = ROWS * 128 * 2            # bytes of one [10, 128] BF16 tensor
BASE = 0x7F0000000000           # fake device addresses, 4 KiB apart


def addr(k):
    return BASE + k * 0x10000


X, G, W, DY, Y, DX, DG, DW, WS = (addr(k) for k in range(9))
WS_BYTES = 32768 + 2048         # counters + chunk and group partials (10 rows, D <= 256)


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gated_rmsnorm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert len(names) == 12, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
    assert sorted(binding._SIGS) == names


def test_workspace_bytes(lib):
    C = lib.gated_rmsnorm_workspace_init_bytes()
    assert C == 32768
    assert lib.gated_rmsnorm_chunk_rows(0, 128, 0) == 0
    assert lib.gated_rmsnorm_chunk_rows(10, 96, 0) == 0
    assert lib.gated_rmsnorm_chunk_rows(10, 128, 3) == 0
    for rows in (1, 49488, 196608, 12582912):
        for dt in (0, 1, 2):
            assert lib.gated_rmsnorm_chunk_rows(rows, 128, dt) == 128
            assert lib.gated_rmsnorm_chunk_rows(rows, 256, dt) == 128
        # 128-byte rows (D = 64, 16-bit) take 256-row chunks
        assert lib.gated_rmsnorm_chunk_rows(rows, 64, 0) == 256
        assert lib.gated_rmsnorm_chunk_rows(rows, 64, 1) == 256
        assert lib.gated_rmsnorm_chunk_rows(rows, 64, 2) == 128

    def expect(rows, D=128):
        R = 128   # the size allocated covers the smallest chunks of any type
        chunks = math.ceil(rows / R)
        gs = math.isqrt(chunks - 1) + 1 if chunks > 1 else 1   # ceil(sqrt(chunks))
        return C + (chunks + math.ceil(chunks / gs)) * 4 * D

    assert lib.gated_rmsnorm_workspace_bytes(0, 128) == 0
    assert lib.gated_rmsnorm_workspace_bytes(-5, 128) == 0
    for bad_d in (0, 32, 96, 127, 192, 512):
        assert lib.gated_rmsnorm_workspace_bytes(10, bad_d) == 0
    assert lib.gated_rmsnorm_workspace_bytes(1, 128) == C + 1024
    assert lib.gated_rmsnorm_workspace_bytes(128, 128) == C + 1024
    assert lib.gated_rmsnorm_workspace_bytes(129, 128) == C + 3 * 512
    for rows in (5 * 128, 17 * 128 + 3, 49488, 196607, 196608, 368832, 1572864, 12582912,
                 2**31 - 1):
        for D in (64, 128, 256):
            assert lib.gated_rmsnorm_workspace_bytes(rows, D) == expect(rows, D), (rows, D)
    assert lib.gated_rmsnorm_workspace_bytes(2**31, 128) == 0


def test_status_strings(lib):
    for code in range(10):
        s = lib.gated_rmsnorm_status_string(code).decode()
        assert s.startswith("GRN_"), s
    assert "unknown" in lib.gated_rmsnorm_status_string(99).decode()


def fwd(lib, x=X, g=G, w=W, y=Y, rows=ROWS, D=128, eps=1e-6, dtype=0):
    return lib.gated_rmsnorm_fwd(x, g, w, y, rows, D, eps, dtype, None)


def bwd(lib, x=X, g=G, w=W, dy=DY, dx=DX, dg=DG, dw=DW, ws=WS, ws_bytes=WS_BYTES,
        rows=ROWS, D=128, eps=1e-6, dtype=0, dw_fp32=1):
    return lib.gated_rmsnorm_bwd(x, g, w, dy, dx, dg, dw, ws, ws_bytes, rows, D,
                                 eps, dtype, dw_fp32, None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=0), SHAPE), (dict(D=32), SHAPE), (dict(D=127), SHAPE), (dict(D=512), SHAPE),
    (dict(rows=-1), SHAPE), (dict(rows=2**31), SHAPE), (dict(dtype=-1), DTYPE),
    (dict(dtype=3), DTYPE), (dict(eps=float("nan")), EPS), (dict(x=None), NULL),
    (dict(w=None), NULL), (dict(y=X), ALIAS), (dict(y=W), ALIAS), (dict(y=G + 16), ALIAS),
    (dict(x=X + 8), ALIGN), (dict(w=W + 4, dtype=2), ALIGN),
    # a [10, 256] FP32 y 10 KiB long reaches into x placed 8 KiB after it
    (dict(D=256, dtype=2, y=X - 8192), ALIAS),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def ckpt(lib, y=Y, **kw):
    a = dict(x=X, g=G, w=W, dy=DY, dx=DX, dg=DG, dw=DW, ws=WS, ws_bytes=WS_BYTES,
             rows=ROWS, D=128, eps=1e-6, dtype=0, dw_fp32=1)
    a.update(kw)
    return lib.gated_rmsnorm_ckpt_step(a["x"], a["g"], a["w"], a["dy"], y, a["dx"],
                                       a["dg"], a["dw"], a["ws"], a["ws_bytes"],
                                       a["rows"], a["D"], a["eps"], a["dtype"],
                                       a["dw_fp32"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=192), SHAPE), (dict(D=512), SHAPE), (dict(dtype=3), DTYPE), (dict(dw_fp32=2), DTYPE),
    (dict(dw_fp32=-1), DTYPE), (dict(eps=-0.5), EPS),
    (dict(ws_bytes=0), WORKSPACE), (dict(ws_bytes=511), WORKSPACE),
    (dict(ws=None), WORKSPACE),
    (dict(dy=None), NULL), (dict(dx=None), NULL), (dict(dg=None), NULL), (dict(dw=None), NULL),
    (dict(dy=DY + 8), ALIGN), (dict(dw=DW + 2, dw_fp32=1), ALIGN), (dict(dw=DW + 1, dw_fp32=0), ALIGN),
    (dict(ws=WS + 4), ALIGN),
    # FP32 dw of FP16 inputs, FP32 dw of FP32 inputs: 4-byte aligned
    (dict(dtype=1, dw=DW + 2, dw_fp32=1), ALIGN), (dict(dtype=2, dw=DW + 2, dw_fp32=0), ALIGN),
    (dict(dtype=1, dw=DW + 1, dw_fp32=0), ALIGN),
    (dict(D=64, ws_bytes=32768 + 511), WORKSPACE), (dict(D=256, ws_bytes=32768 + 2047), WORKSPACE),
    (dict(dx=X), ALIAS), (dict(dx=DY + 32), ALIAS), (dict(dg=DX), ALIAS),
    (dict(dw=DX + 64), ALIAS), (dict(ws=DG + 256), ALIAS), (dict(dw=WS + 128), ALIAS),
    (dict(dw=W), ALIAS),
])
def test_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(y=None), NULL), (dict(y=DX), ALIAS), (dict(y=DW), ALIAS), (dict(y=X + 32), ALIAS),
    (dict(y=WS), ALIAS), (dict(dw_fp32=5), DTYPE), (dict(ws_bytes=100), WORKSPACE),
    (dict(D=1), SHAPE), (dict(eps=float("-inf")), EPS),
])
def test_ckpt_rejects(lib, kw, code):
    assert ckpt(lib, **kw) == code


def fwd_s(lib, x=X, sx=128, g=G, sg=128, w=W, y=Y, sy=128, rows=ROWS, D=128, eps=1e-6,
          dtype=0):
    return lib.gated_rmsnorm_fwd_strided(x, sx, g, sg, w, y, sy, rows, D, eps, dtype, None)


def bwd_s(lib, x=X, sx=128, g=G, sg=128, w=W, dy=DY, sdy=128, dx=DX, sdx=128, dg=DG,
          sdg=128, dw=DW, ws=WS, ws_bytes=WS_BYTES, rows=ROWS, eps=1e-6, dw_fp32=1, det=1):
    return lib.gated_rmsnorm_bwd_strided(x, sx, g, sg, w, dy, sdy, dx, sdx, dg, sdg, dw, ws,
                                         ws_bytes, rows, 128, eps, 0, dw_fp32, det, None)


def ckpt_s(lib, det=1, dw_fp32=1, y=Y):
    return lib.gated_rmsnorm_ckpt_step_strided(X, 128, G, 128, W, DY, 128, y, 128, DX, 128,
                                               DG, 128, DW, WS, WS_BYTES, ROWS, 128, 1e-6, 0,
                                               dw_fp32, det, None)


@pytest.mark.parametrize("kw,code", [
    (dict(sx=64), SHAPE), (dict(sg=127), SHAPE), (dict(sy=0), SHAPE), (dict(sx=-128), SHAPE),
    (dict(sx=(1 << 24) + 8), SHAPE), (dict(sx=132), ALIGN), (dict(sy=136 + 4), ALIGN),
    (dict(x=None), NULL),
    # y rows interleaved with x's rows (same pitch) but sharing 16 bytes per row
    (dict(sx=256, sy=256, y=X + 240), ALIAS),
    # y overlapping g with a different pitch (conservative range test)
    (dict(sg=256, sy=384, y=G + 256), ALIAS),
    # rows stay 16-byte aligned: 4-element steps for FP32, 8 for FP16
    (dict(dtype=2, sx=130), ALIGN), (dict(dtype=1, sg=132), ALIGN), (dict(D=64, sy=60), SHAPE),
    (dict(D=256, sx=248), SHAPE),
    # FP32 rows of 512 bytes: y at x + 256 bytes shares half of each row of x
    (dict(dtype=2, sx=256, sy=256, y=X + 256), ALIAS),
])
def test_fwd_strided_rejects(lib, kw, code):
    assert fwd_s(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(sdx=120), SHAPE), (dict(sdg=204), ALIGN),
    # dx and dg as the halves of one buffer, but dg starting 16 bytes too early
    (dict(sdx=256, sdg=256, dg=DX + 240), ALIAS),
    # dg written over dy's rows
    (dict(sdy=256, sdg=256, dg=DY), ALIAS),
    (dict(sx=256, sdx=256, dx=X + 128), ALIAS),
    (dict(det=2), ARG), (dict(det=-1), ARG), (dict(det=0, dw_fp32=3), DTYPE),
    (dict(det=0, dx=None), NULL), (dict(det=0, ws_bytes=100), WORKSPACE),
])
def test_bwd_strided_rejects(lib, kw, code):
    assert bwd_s(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(det=2), ARG), (dict(det=0, y=None), NULL), (dict(det=0, dw_fp32=7), DTYPE),
])
def test_ckpt_strided_rejects(lib, kw, code):
    assert ckpt_s(lib, **kw) == code


def test_workspace_init_rejects(lib):
    C = lib.gated_rmsnorm_workspace_init_bytes()
    assert lib.gated_rmsnorm_workspace_init(None, C, None) == NULL
    assert lib.gated_rmsnorm_workspace_init(WS, C - 4, None) == WORKSPACE
    assert lib.gated_rmsnorm_workspace_init(WS + 8, C, None) == ALIGN


def test_binding_rejects_cpu_tensors():
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    w = torch.ones(128, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        binding.gated_rmsnorm_fwd(x, x, w)
    with pytest.raises(TypeError):
        binding.gated_rmsnorm_bwd(x, x, w, x)


def test_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        binding.load_library(tmp_path / "nope.so")


def test_noalloc_rejects_before_any_launch(lib):
    """gated_rmsnorm_bwd_noalloc checks every argument, and that the call
    fits the static scratch (GRN_NOALLOC_SCRATCH_BYTES = 64 MiB), before any
    HIP call: these fake pointers are never touched."""
    f = lib.gated_rmsnorm_bwd_noalloc
    eps = 1e-6
    header = HEADER.read_text()
    assert "#define GRN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in header
    cap = 64 << 20
    # the largest BF16 D = 128 call that fits, and the first that does not
    C = lib.gated_rmsnorm_workspace_init_bytes()

    def need(rows, D=128, R=128):
        chunks = math.ceil(rows / R)
        gs = math.isqrt(chunks - 1) + 1 if chunks > 1 else 1
        return C + (chunks + math.ceil(chunks / gs)) * 4 * D

    lo, hi = 1, 1 << 26
    while lo < hi:                       # largest rows with need(rows) <= cap
        mid = (lo + hi + 1) // 2
        if need(mid) <= cap:
            lo = mid
        else:
            hi = mid - 1
    assert 16_000_000 < lo < 17_000_000
    assert f(X, G, W, DY, DX, DG, DW, lo + 1, 128, eps, 0, 0, None) == SCRATCH
    assert f(X, G, W, DY, DX, DG, DW, 12582912 * 2, 128, eps, 0, 1, None) == SCRATCH
    # D = 256 needs twice the bytes per chunk
    assert f(X, G, W, DY, DX, DG, DW, lo, 256, eps, 0, 0, None) == SCRATCH
    assert f(X, G, W, DY, DX, DG, DW, 10, 96, eps, 0, 0, None) == SHAPE
    assert f(X, G, W, DY, DX, DG, DW, -1, 128, eps, 0, 0, None) == SHAPE
    assert f(X, G, W, DY, DX, DG, DW, 10, 128, eps, 7, 0, None) == DTYPE
    assert f(X, G, W, DY, DX, DG, DW, 10, 128, eps, 0, 2, None) == DTYPE
    assert f(X, G, W, DY, DX, DG, DW, 10, 128, -1.0, 0, 0, None) == EPS
    assert f(X, G, None, DY, DX, DG, DW, 10, 128, eps, 0, 0, None) == NULL
    assert f(X, G, W, DY, DX, DG, None, 10, 128, eps, 0, 0, None) == NULL
    assert f(X, G, W, DY, X, DG, DW, 10, 128, eps, 0, 0, None) == ALIAS
    assert f(X + 8, G, W, DY, DX, DG, DW, 10, 128, eps, 0, 0, None) == ALIGN
    assert b"GRN_ERR_SCRATCH" in lib.gated_rmsnorm_status_string(SCRATCH)


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

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, WORKSPACE, EPS, HIP = range(9)
ROWS = 10
ACT = ROWS * 128 * 2            # bytes of one [10, 128] BF16 tensor
BASE = 0x7F0000000000           # fake device addresses, 4 KiB apart


def addr(k):
    return BASE + k * 0x10000


X, G, W, DY, Y, DX, DG, DW, WS = (addr(k) for k in range(9))
WS_BYTES = 32768 + 512 + 512    # counters + 1 chunk partial + 1 group partial


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gated_rmsnorm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert len(names) == 8, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
    assert sorted(binding._SIGS) == names


def test_workspace_bytes(lib):
    R = lib.gated_rmsnorm_chunk_rows()
    C = lib.gated_rmsnorm_workspace_init_bytes()
    assert R == 128 and C == 32768

    def expect(rows):
        chunks = math.ceil(rows / R)
        gs = math.isqrt(chunks - 1) + 1 if chunks > 1 else 1   # ceil(sqrt(chunks))
        return C + (chunks + math.ceil(chunks / gs)) * 512

    assert lib.gated_rmsnorm_workspace_bytes(0, 128) == 0
    assert lib.gated_rmsnorm_workspace_bytes(-5, 128) == 0
    assert lib.gated_rmsnorm_workspace_bytes(10, 64) == 0
    assert lib.gated_rmsnorm_workspace_bytes(1, 128) == C + 1024
    assert lib.gated_rmsnorm_workspace_bytes(R, 128) == C + 1024
    assert lib.gated_rmsnorm_workspace_bytes(R + 1, 128) == C + 3 * 512
    for rows in (5 * R, 17 * R + 3, 368832, 1572864, 12582912, 2**31 - 1):
        assert lib.gated_rmsnorm_workspace_bytes(rows, 128) == expect(rows), rows
    assert lib.gated_rmsnorm_workspace_bytes(2**31, 128) == 0


def test_status_strings(lib):
    for code in range(9):
        s = lib.gated_rmsnorm_status_string(code).decode()
        assert s.startswith("GRN_"), s
    assert "unknown" in lib.gated_rmsnorm_status_string(99).decode()


def fwd(lib, x=X, g=G, w=W, y=Y, rows=ROWS, D=128, eps=1e-6, dtype=0):
    return lib.gated_rmsnorm_fwd(x, g, w, y, rows, D, eps, dtype, None)


def bwd(lib, x=X, g=G, w=W, dy=DY, dx=DX, dg=DG, dw=DW, ws=WS, ws_bytes=WS_BYTES,
        rows=ROWS, D=128, eps=1e-6, dtype=0, dw_fp32=1):
    return lib.gated_rmsnorm_bwd(x, g, w, dy, dx, dg, dw, ws, ws_bytes, rows, D,
                                 eps, dtype, dw_fp32, None)


def ckpt(lib, y=Y, **kw):
    a = dict(x=X, g=G, w=W, dy=DY, dx=DX, dg=DG, dw=DW, ws=WS, ws_bytes=WS_BYTES,
             rows=ROWS, D=128, eps=1e-6, dtype=0, dw_fp32=1)
    a.update(kw)
    return lib.gated_rmsnorm_ckpt_step(a["x"], a["g"], a["w"], a["dy"], y, a["dx"],
                                       a["dg"], a["dw"], a["ws"], a["ws_bytes"],
                                       a["rows"], a["D"], a["eps"], a["dtype"],
                                       a["dw_fp32"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=256), SHAPE), (dict(dtype=3), DTYPE), (dict(dw_fp32=2), DTYPE),
    (dict(dw_fp32=-1), DTYPE), (dict(eps=-0.5), EPS),
    (dict(ws_bytes=0), WORKSPACE), (dict(ws_bytes=511), WORKSPACE),
    (dict(ws=None), WORKSPACE),
    (dict(dy=None), NULL), (dict(dx=None), NULL), (dict(dg=None), NULL), (dict(dw=None), NULL),
    (dict(dy=DY + 8), ALIGN), (dict(dw=DW + 2, dw_fp32=1), ALIGN), (dict(dw=DW + 1, dw_fp32=0), ALIGN),
    (dict(ws=WS + 4), ALIGN),
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

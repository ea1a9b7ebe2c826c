"""FP16 and FP32 storage and row widths D = 64, 128, 256 on the GPU.

The same kernels, instantiated per element type and width, against the FP64
oracle on the exact values of the inputs (FP16 and FP32 widen to FP64
exactly).  Bars: y, dx, dg within 1e-2 (BF16), 2e-3 (FP16) or 1e-3 (FP32) of
the oracle under the per-row floor; FP32 dw relative 1e-4; BF16/FP16 dw
within 2 ulp of the nearest value to the exact sum.  Rows are chosen to
leave a ragged tail for every tiling (a wave access spans 8, 4, 2 or 1 rows
depending on the width and type).
"""
import numpy as np
import pytest
import torch

import oracle
from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import WORKLOADS, make_inputs, make_workload_inputs

from _compare import (DW32_TOL, DW16_ULPS, Y_TOL, Y_TOL_F16, Y_TOL_F32, act_err, dw16_check,
                      dw32_err, dwf16_check)
from gpu_util import bits, say

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
BARS = {torch.bfloat16: Y_TOL, torch.float16: Y_TOL_F16, torch.float32: Y_TOL_F32}


def _f64(t):
    if t.dtype == torch.bfloat16:
        return oracle.bf16_to_f64(bits(t))
    return t.detach().cpu().double().numpy()


def _oracle(inp, eps):
    a = {k: np.ascontiguousarray(_f64(v)) for k, v in inp.items()}
    y = oracle.fwd(a["x"], a["g"], a["w"], eps)
    dx, dg, dw = oracle.bwd(a["x"], a["g"], a["w"], a["dy"], eps)
    return y, dx, dg, dw


def _check_acts(dtype, got, ref):
    errs = []
    for name, t, r in zip(("y", "dx", "dg"), got, ref):
        err, _, _ = act_err(_f64(t), r)
        errs.append(err)
        assert err <= BARS[dtype], f"{name}: rel err {err:.3e} > {BARS[dtype]:.0e}"
    say("  y/dx/dg max rel err " + " ".join(f"{e:.2e}" for e in errs))


def _check_dw(dw, ref, dtype, dw_fp32):
    if dw_fp32 or dtype == torch.float32:
        assert dw.dtype == torch.float32
        e = dw32_err(_f64(dw), ref)
        assert e <= DW32_TOL, f"dw fp32 rel err {e:.3e}"
        return
    assert dw.dtype == dtype
    if dtype == torch.bfloat16:
        worst, ok = dw16_check(bits(dw), ref)
    else:
        worst, ok = dwf16_check(dw.cpu().numpy().view(np.uint16), ref)
    assert ok, f"dw off by {worst} ulp (allowed {DW16_ULPS})"


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dname", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows", [1, 37, 4099])
def test_dtype_width_parity(dname, D, rows):
    dtype = DTYPES[dname]
    say(f"[dtypes] {dname} D={D} rows={rows}")
    inp = make_inputs(rows, D, seed=100 + rows + D, device="cuda", dtype=dtype)
    y_ref, dx_ref, dg_ref, dw_ref = _oracle(inp, 1e-6)
    y = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], 1e-6)
    for dw_fp32 in (False, True):
        dx, dg, dw = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"],
                                               1e-6, dw_fp32=dw_fp32)
        torch.cuda.synchronize()
        assert y.dtype == dx.dtype == dg.dtype == dtype
        _check_acts(dtype, (y, dx, dg), (y_ref, dx_ref, dg_ref))
        _check_dw(dw, dw_ref, dtype, dw_fp32)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dname", ["bf16", "f16", "f32"])
def test_dtype_width_paths(dname, D):
    """Checkpointed step, non-deterministic dw and strided rows reach the
    same instantiations: step equals fwd + bwd bitwise, strided rows equal
    packed rows bitwise, non-deterministic dw meets the dw bar."""
    dtype = DTYPES[dname]
    rows = 3001
    say(f"[dtypes] paths {dname} D={D} rows={rows}")
    inp = make_inputs(rows, D, seed=7, device="cuda", dtype=dtype)
    x, g, w, dy = inp["x"], inp["g"], inp["w"], inp["dy"]
    _, _, _, dw_ref = _oracle(inp, 1e-6)
    y = binding.gated_rmsnorm_fwd(x, g, w, 1e-6)
    dx, dg, dw = binding.gated_rmsnorm_bwd(x, g, w, dy, 1e-6, dw_fp32=True)
    y2, dx2, dg2, dw2 = binding.gated_rmsnorm_ckpt_step(x, g, w, dy, 1e-6, True)
    _, _, dw3 = binding.gated_rmsnorm_bwd(x, g, w, dy, 1e-6, True, deterministic=False)
    xg = torch.empty(rows, 2 * D, dtype=dtype, device="cuda")
    xg[:, :D] = x
    xg[:, D:] = g
    out = torch.full((rows, 2 * D), 7.0, dtype=dtype, device="cuda")
    dx4, dg4, dw4 = binding.gated_rmsnorm_bwd(xg[:, :D], xg[:, D:], w, dy, 1e-6, True,
                                              dx=out[:, :D], dg=out[:, D:])
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(a.contiguous().view(torch.uint8),  # noqa: E731
                                    b.contiguous().view(torch.uint8))
    assert same(y, y2) and same(dx, dx2) and same(dg, dg2) and same(dw, dw2)
    assert same(dx, dx4) and same(dg, dg4) and same(dw, dw4)
    _check_dw(dw3, dw_ref, dtype, True)


def test_16384x32_full_size():
    """The H = 32 shape of the pages' tables at full size: sampled rows of
    y, dx, dg and the whole dw against the oracle (BF16, D = 128)."""
    wl = WORKLOADS["16384x32"]
    say(f"[dtypes] {wl.name} rows={wl.rows}")
    inp = make_workload_inputs(wl, device="cuda")
    y = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], wl.eps)
    dx, dg, dw = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], wl.eps,
                                           dw_fp32=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([np.arange(300), np.arange(wl.rows - 300, wl.rows),
                                    rng.integers(0, wl.rows, 2000)]))
    ti = torch.from_numpy(idx).cuda()
    sub = {k: (v[ti] if k != "w" else v) for k, v in inp.items()}
    y_ref, dx_ref, dg_ref, _ = _oracle(sub, wl.eps)
    _check_acts(torch.bfloat16, (y[ti], dx[ti], dg[ti]), (y_ref, dx_ref, dg_ref))
    b = {k: bits(v) for k, v in inp.items()}
    _, _, dw_ref = oracle.bwd(b["x"], b["g"], b["w"], b["dy"], wl.eps)
    _check_dw(dw, dw_ref, torch.bfloat16, True)


# Tensors of 256 MiB and more take the large-tensor backward; FP32 holds
# back its last step's stores there, FP16 and BF16 at D = 256 do not.  Row
# counts leave a ragged last chunk.
@pytest.mark.parametrize("dname,D,rows", [("f32", 256, 270001), ("f16", 128, 1050001),
                                          ("bf16", 256, 530001)])
def test_large_tensor_types(dname, D, rows):
    """Sampled rows of y, dx, dg and the whole dw (both dw types) against
    the oracle for the large-tensor kernels of other types and widths."""
    dtype = DTYPES[dname]
    say(f"[dtypes] large {dname} D={D} rows={rows}")
    inp = make_inputs(rows, D, seed=11, device="cuda", dtype=dtype)
    y = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], 1e-6)
    outs = {}
    for dw_fp32 in (False, True):
        outs[dw_fp32] = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"],
                                                  1e-6, dw_fp32=dw_fp32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    idx = np.unique(np.concatenate([np.arange(200), np.arange(rows - 300, rows),
                                    rng.integers(0, rows, 1500)]))
    ti = torch.from_numpy(idx).cuda()
    sub = {k: (v[ti] if k != "w" else v) for k, v in inp.items()}
    y_ref, dx_ref, dg_ref, _ = _oracle(sub, 1e-6)
    for dw_fp32, (dx, dg, _) in outs.items():
        _check_acts(dtype, (y[ti], dx[ti], dg[ti]), (y_ref, dx_ref, dg_ref))
    a = {k: np.ascontiguousarray(_f64(v)) for k, v in inp.items()}
    _, _, dw_ref = oracle.bwd(a["x"], a["g"], a["w"], a["dy"], 1e-6)
    del a
    for dw_fp32, (_, _, dw) in outs.items():
        _check_dw(dw, dw_ref, dtype, dw_fp32)


def test_f16_outputs_beyond_range_are_infinite():
    """FP16 storage: a y whose exact value lies beyond FP16's range (>= 65520
    after rounding) comes out infinite with the right sign, the rest of the
    row stays finite and within the bar."""
    rows, D = 4, 128
    say(f"[dtypes] f16 overflow rows={rows}")
    inp = make_inputs(rows, D, seed=77, device="cuda", dtype=torch.float16)
    g = inp["g"].clone()
    w = inp["w"].clone()
    g[0, :8] = 400.0       # silu(400) = 400
    w[:8] = 300.0          # |y| ~ |n| * 1.2e5 for the first 8 columns of row 0
    inp = {"x": inp["x"], "g": g, "w": w, "dy": inp["dy"]}
    y = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], 1e-6)
    torch.cuda.synchronize()
    y_ref, _, _, _ = _oracle(inp, 1e-6)
    got = _f64(y)
    big = np.abs(y_ref) >= 65520.0
    assert big.any()
    assert np.all(np.isinf(got[big])) and np.all(np.sign(got[big]) == np.sign(y_ref[big]))
    rest = ~big
    assert np.all(np.isfinite(got[rest]))
    err = np.max(np.abs(got[rest] - y_ref[rest]) / np.maximum(np.abs(y_ref[rest]), 1e-3))
    assert err <= Y_TOL_F16, err

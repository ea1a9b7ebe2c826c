"""Shared plumbing of the GPU tests: run the HIP path, run the oracle, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import bf16_bits

from _compare import DW16_ULPS, DW32_TOL, Y_TOL, act_err, dw16_check, dw32_err


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(*a, file=sys.stderr, flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return bf16_bits(t)


def f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.bf16_to_f64(bf16_bits(t))
    return t.detach().cpu().double().numpy()


def gpu_all(inp, eps, dw_fp32):
    """Forward then backward through the C ABI; returns GPU tensors."""
    y = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], eps)
    dx, dg, dw = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], eps,
                                           dw_fp32=dw_fp32)
    torch.cuda.synchronize()
    return y, dx, dg, dw


def oracle_all(inp, eps, want_dw=True):
    b = {k: bits(v) for k, v in inp.items()}
    y = oracle.fwd(b["x"], b["g"], b["w"], eps)
    dx, dg, dw = oracle.bwd(b["x"], b["g"], b["w"], b["dy"], eps, want_dw=want_dw)
    return y, dx, dg, dw


def assert_acts_close(name, gpu_t, ref):
    err, binds, unf = act_err(f64(gpu_t), ref)
    assert err <= Y_TOL, f"{name}: max rel err {err:.3e} (floor binds {binds}, unfloored {unf:.3e})"
    return err


def assert_dw_close(dw_t, ref, dw_fp32):
    if dw_fp32:
        assert dw_t.dtype == torch.float32
        e = dw32_err(f64(dw_t), ref)
        assert e <= DW32_TOL, f"dw fp32 rel err {e:.3e}"
        return e
    assert dw_t.dtype == torch.bfloat16
    worst, ok = dw16_check(bits(dw_t), ref)
    assert ok, f"dw bf16 off by {worst} ulp (allowed {DW16_ULPS})"
    return worst


def oracle_dw_streamed(inp, eps, chunk=1 << 20):
    """Oracle dw over every row, in row chunks whose FP64 sums are added in order."""
    rows = inp["x"].shape[0]
    w = bits(inp["w"])
    dw = np.zeros(128)
    for r0 in range(0, rows, chunk):
        sl = slice(r0, min(rows, r0 + chunk))
        _, _, part = oracle.bwd(bits(inp["x"][sl]), bits(inp["g"][sl]), w,
                                bits(inp["dy"][sl]), eps)
        dw += part
    return dw

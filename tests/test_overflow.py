"""Rows whose sum of squares exceeds FP32's range, against the FP64 oracle.

The definition (flashinfer PR #8701 names the operator; r = 1/sqrt(mean(x^2)
+ eps)) has no range limit, and BF16 or FP32 inputs can hold entries up to
about 3.4e38, whose squares do not fit FP32.  Rows with entries at 1e20 and
1e30 (and 1e36 in FP32 storage) are placed among ordinary rows, in every
backward shape that can meet them: the small-tensor and the middle shape
(chunks in interleaved windows), the prefetching shape whose last step's
stores are held back (BF16, D = 64, from 256 MiB per tensor), FP32
storage, the non-deterministic dw and the checkpointed step whose recomputed
forward runs inside the backward's launch.  Checked:

* y, dx and dg of those rows (and of sampled ordinary rows) and the whole dw
  against the oracle, under the usual bars;
* every ordinary row's y, dx and dg bitwise equal to a run in which the huge
  rows were replaced by ordinary values (a row's result depends on that row
  only);
* dw bitwise equal over two runs.
"""
import numpy as np
import pytest
import torch

import oracle
from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import make_inputs

from _compare import DW32_TOL, Y_TOL, Y_TOL_F32, act_err, dw16_check, dw32_err
from gpu_util import bits, say

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _f64(t):
    if t.dtype == torch.bfloat16:
        return oracle.bf16_to_f64(bits(t))
    return t.detach().cpu().double().numpy()


def _host(t):
    """Oracle input: BF16 bit patterns, or FP64 values of other types."""
    if t.dtype == torch.bfloat16:
        return np.ascontiguousarray(bits(t))
    return np.ascontiguousarray(t.detach().cpu().double().numpy())


def _oracle_rows(inp, idx):
    sub = {k: (_host(v[idx]) if k != "w" else _host(v)) for k, v in inp.items()}
    y = oracle.fwd(sub["x"], sub["g"], sub["w"], EPS)
    dx, dg, _ = oracle.bwd(sub["x"], sub["g"], sub["w"], sub["dy"], EPS, want_dw=False)
    return y, dx, dg


def _oracle_dw(inp, chunk=1 << 20):
    rows, D = inp["x"].shape
    w = _host(inp["w"])
    dw = np.zeros(D)
    for r0 in range(0, rows, chunk):
        sl = slice(r0, min(rows, r0 + chunk))
        _, _, part = oracle.bwd(_host(inp["x"][sl]), _host(inp["g"][sl]), w,
                                _host(inp["dy"][sl]), EPS)
        dw += part
    return dw


def _huge_rows(rows, D, R):
    """Rows to scale: both ends, every lane position of a wave step in some
    chunk, several rows of one wave, and the last step of a chunk (held
    stores where the shape holds them)."""
    rng = np.random.default_rng(rows)
    picks = {0, 1, rows - 1, rows - 2}
    for c in (3, 7):
        base = c * R
        picks.update(base + o for o in (0, 5, R // 2 + 2, R // 2 + 9, R - 1) if base + o < rows)
    picks.update(int(v) for v in rng.integers(0, rows, 40))
    return np.array(sorted(picks))


def _run(inp, dw_fp32, det, ckpt):
    x, g, w, dy = inp["x"], inp["g"], inp["w"], inp["dy"]
    if ckpt:
        y, dx, dg, dw = binding.gated_rmsnorm_ckpt_step(x, g, w, dy, EPS, dw_fp32=dw_fp32,
                                                        deterministic=det)
    else:
        y = binding.gated_rmsnorm_fwd(x, g, w, EPS)
        dx, dg, dw = binding.gated_rmsnorm_bwd(x, g, w, dy, EPS, dw_fp32=dw_fp32,
                                               deterministic=det)
    torch.cuda.synchronize()
    return y, dx, dg, dw


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


CASES = [
    # (name, dtype, D, rows, scales, deterministic, checkpointed step)
    ("bf16 small", torch.bfloat16, 128, 5003, (1e20, 1e30), True, False),
    ("bf16 small ckpt", torch.bfloat16, 128, 5003, (1e20, 1e30), True, True),
    ("bf16 middle", torch.bfloat16, 128, 140001, (1e20, 1e30), True, False),
    ("bf16 middle nondet", torch.bfloat16, 128, 140001, (1e20, 1e30), False, False),
    ("bf16 D=64 prefetching, held", torch.bfloat16, 64, 2200001, (1e20, 1e30), True, False),
    ("f32 small", torch.float32, 128, 3001, (1e20, 1e30, 1e36), True, False),
    ("f32 middle", torch.float32, 128, 70001, (1e20, 1e30, 1e36), True, False),
    ("bf16 D=256 middle", torch.bfloat16, 256, 70001, (1e20, 1e30), True, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rows_beyond_fp32_squares(case):
    name, dtype, D, rows, scales, det, ckpt = case
    say(f"[overflow] {name}: rows={rows} D={D} scales={scales}")
    R = binding.load_library().gated_rmsnorm_chunk_rows(
        rows, D, {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}[dtype])
    base = make_inputs(rows, D, seed=rows % 977, device="cuda", dtype=dtype)
    huge = _huge_rows(rows, D, R)
    inp = dict(base)
    x = base["x"].float().clone()
    sc = torch.tensor([scales[k % len(scales)] for k in range(huge.size)], device="cuda")
    hi = torch.from_numpy(huge).cuda()
    x[hi] = x[hi] * sc[:, None]
    x[hi[0], 0] = 3.0 * scales[-1]          # one entry far above the rest of its row
    inp["x"] = x.to(dtype)
    assert torch.isfinite(inp["x"]).all()
    bar = Y_TOL if dtype == torch.bfloat16 else Y_TOL_F32
    for dw_fp32 in ((True, False) if dtype == torch.bfloat16 else (True,)):
        y, dx, dg, dw = _run(inp, dw_fp32, det, ckpt)
        for t in (y, dx, dg):
            assert torch.isfinite(t).all().item()
        # the huge rows and sampled ordinary rows against the oracle
        rng = np.random.default_rng(3)
        idx_np = np.unique(np.concatenate([huge, rng.integers(0, rows, 1500)]))
        idx = torch.from_numpy(idx_np).cuda()
        y_ref, dx_ref, dg_ref = _oracle_rows(inp, idx)
        for nm, t, r in (("y", y, y_ref), ("dx", dx, dx_ref), ("dg", dg, dg_ref)):
            err, _, _ = act_err(_f64(t[idx]), r)
            assert err <= bar, f"{nm}: rel err {err:.3e} > {bar:.0e}"
        dw_ref = _oracle_dw(inp)
        if dw_fp32 or dtype == torch.float32:
            e = dw32_err(_f64(dw), dw_ref)
            assert e <= DW32_TOL, f"dw rel err {e:.3e}"
        else:
            worst, ok = dw16_check(bits(dw), dw_ref)
            assert ok, f"dw off by {worst} ulp"
        if det:
            dw_again = _run(inp, dw_fp32, det, ckpt)[3]
            assert _same(dw, dw_again)
        # ordinary rows: bitwise those of a run without the huge rows
        y0, dx0, dg0, _ = _run(base, dw_fp32, det, ckpt)
        keep = torch.ones(rows, dtype=torch.bool, device="cuda")
        keep[hi] = False
        for a, b in ((y, y0), (dx, dx0), (dg, dg0)):
            assert _same(a[keep], b[keep])
        del y, dx, dg, y0, dx0, dg0

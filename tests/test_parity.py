"""GPU parity: the HIP path against the FP64 oracle, element by element.

Small and ragged row counts (spanning several workgroup tiles, dw chunks and
a partial tail), the 1031x48 workload in full, special values, empty input,
and the four larger workloads at full size on sampled rows (y, dx, dg) with
dw against the oracle's sum over every row.  Tolerances are in _compare.py.
"""
import numpy as np
import pytest
import torch

import oracle
from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import WORKLOADS, make_inputs, make_workload_inputs

from gpu_util import (assert_acts_close, assert_dw_close, bits, f64, gpu_all, oracle_all,
                      oracle_dw_streamed, say)

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.mark.parametrize("rows", [1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255,
                                  256, 257, 511, 513, 1000, 4099, 12345,
                                  196607, 196608, 196609])
def test_small_and_ragged(rows):
    say(f"[parity] ragged rows={rows}")
    inp = make_inputs(rows, seed=rows, device="cuda")
    y_ref, dx_ref, dg_ref, dw_ref = oracle_all(inp, EPS)
    for dw_fp32 in (True, False):
        y, dx, dg, dw = gpu_all(inp, EPS, dw_fp32)
        assert_acts_close("y", y, y_ref)
        assert_acts_close("dx", dx, dx_ref)
        assert_acts_close("dg", dg, dg_ref)
        assert_dw_close(dw, dw_ref, dw_fp32)


def test_workload_1031x48_full():
    wl = WORKLOADS["1031x48"]
    say(f"[parity] {wl.name} rows={wl.rows} full")
    inp = make_workload_inputs(wl, device="cuda")
    y_ref, dx_ref, dg_ref, dw_ref = oracle_all(inp, wl.eps)
    for dw_fp32 in (False, True):
        y, dx, dg, dw = gpu_all(inp, wl.eps, dw_fp32)
        ey = assert_acts_close("y", y, y_ref)
        ex = assert_acts_close("dx", dx, dx_ref)
        eg = assert_acts_close("dg", dg, dg_ref)
        ew = assert_dw_close(dw, dw_ref, dw_fp32)
        say(f"  dw_fp32={dw_fp32}: y {ey:.2e} dx {ex:.2e} dg {eg:.2e} dw {ew}")


def test_empty_rows():
    say("[parity] rows=0")
    x = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    y = binding.gated_rmsnorm_fwd(x, x, w, EPS)
    assert y.shape == (0, 128)
    for dw_fp32 in (True, False):
        dw = torch.full((128,), float("nan"), device="cuda",
                        dtype=torch.float32 if dw_fp32 else torch.bfloat16)
        _, _, dw = binding.gated_rmsnorm_bwd(x, x, w, x, EPS, dw_fp32=dw_fp32, dw=dw)
        torch.cuda.synchronize()
        assert torch.all(dw == 0).item()


def _special_inputs():
    """Rows that exercise the degenerate cases of the operator."""
    rows = 64
    inp = make_inputs(rows, seed=7, device="cpu")
    x = inp["x"].float()
    g = inp["g"].float()
    x[0] = 0.0                      # all-zero row: r = eps^-1/2, y = 0
    x[1] = 3.0                      # constant row
    x[2] = -0.5
    g[3] = 0.0                      # gate zero: y = 0, dg = dy w n / 2
    g[4] = 80.0                     # sigmoid saturates at 1: silu = g
    g[5] = -1000.0                  # sigmoid underflows to 0: y, dx, dg = 0
    g[12] = -80.0                   # sigmoid(-80) ~ 1.8e-35: tiny but not zero
    g[6, ::2] = 1e4
    g[6, 1::2] = -1e4
    x[7] *= 100.0                   # outlier row
    x[8] *= 1e-15                   # tiny row: eps dominates when eps > 0
    x[9, 1:] = 0.0                  # a single non-zero entry
    x[10] *= 1e15                   # large row (mean square 1e30, still FP32)
    x[11, :64] = 0.0                # half of the row zero
    inp["x"] = x.to(torch.bfloat16)
    inp["g"] = g.to(torch.bfloat16)
    return {k: v.cuda() for k, v in inp.items()}


@pytest.mark.parametrize("eps", [1e-6, 1.0, 0.0])
def test_special_values(eps):
    say(f"[parity] special values eps={eps}")
    inp = _special_inputs()
    if eps == 0.0:  # a zero row has no norm without eps; drop it
        inp["x"][0] = 1.0
    y_ref, dx_ref, dg_ref, dw_ref = oracle_all(inp, eps)
    for dw_fp32 in (True, False):
        y, dx, dg, dw = gpu_all(inp, eps, dw_fp32)
        assert_acts_close("y", y, y_ref)
        assert_acts_close("dx", dx, dx_ref)
        assert_acts_close("dg", dg, dg_ref)
        assert_dw_close(dw, dw_ref, dw_fp32)
        yf, dxf, dgf = f64(y), f64(dx), f64(dg)
        assert np.all(yf[3] == 0.0)
        assert np.all(yf[5] == 0.0) and np.all(dxf[5] == 0.0) and np.all(dgf[5] == 0.0)
        if eps > 0:
            assert np.all(yf[0] == 0.0)


def test_every_output_element_written():
    """Outputs pre-filled with NaN: after the call no NaN is left."""
    rows = 1037
    say(f"[parity] NaN-poisoned outputs rows={rows}")
    inp = make_inputs(rows, seed=11, device="cuda")
    nan = lambda: torch.full((rows, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    y, dx, dg = nan(), nan(), nan()
    dw = torch.full((128,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((binding.gated_rmsnorm_workspace_bytes(rows) // 4,), float("nan"),
                    device="cuda")
    binding.gated_rmsnorm_workspace_init(ws)
    binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"], inp["dy"], EPS, True,
                                    y=y, dx=dx, dg=dg, dw=dw, workspace=ws)
    torch.cuda.synchronize()
    for t in (y, dx, dg, dw):
        assert not torch.isnan(t).any().item()


@pytest.mark.parametrize("rows", [70363, 173741])
def test_interleaved_chunks_every_row(rows):
    """The backward takes a chunk's row blocks from windows of 256 chunks.

    70,363 rows (17 MiB per tensor, the small-tensor shape) have 550 chunks:
    two full windows and a last one of 38 chunks whose last chunk holds 91
    rows; 173,741 rows (42 MiB, the middle shape) have 1,358 chunks, a last
    window of 78 and a last chunk of 45 rows.  dx and dg start as NaN: every
    row must be written, and every element must match the oracle, as must
    dw (both types) and dx/dg of the non-deterministic kernel."""
    say(f"[parity] interleaved chunk layout rows={rows}")
    inp = make_inputs(rows, seed=rows % 1000, device="cuda")
    _, dx_ref, dg_ref, dw_ref = oracle_all(inp, EPS)
    for dw_fp32, det in ((True, True), (False, True), (True, False)):
        nan = lambda: torch.full((rows, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        dx, dg = nan(), nan()
        _, _, dw = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], EPS,
                                             dw_fp32=dw_fp32, dx=dx, dg=dg,
                                             deterministic=det)
        torch.cuda.synchronize()
        assert not torch.isnan(dx).any().item() and not torch.isnan(dg).any().item()
        assert_acts_close("dx", dx, dx_ref)
        assert_acts_close("dg", dg, dg_ref)
        assert_dw_close(dw, dw_ref, dw_fp32)


def test_adjacent_buffers_accepted():
    """Inputs and outputs packed back to back in one allocation (no overlap)."""
    rows = 300
    say(f"[parity] adjacent slices rows={rows}")
    inp = make_inputs(rows, seed=12, device="cuda")
    big = torch.empty(6 * rows, 128, dtype=torch.bfloat16, device="cuda")
    x, g, dy, y, dx, dg = (big[k * rows:(k + 1) * rows] for k in range(6))
    x.copy_(inp["x"]); g.copy_(inp["g"]); dy.copy_(inp["dy"])
    binding.gated_rmsnorm_fwd(x, g, inp["w"], EPS, y=y)
    _, _, dw = binding.gated_rmsnorm_bwd(x, g, inp["w"], dy, EPS, True, dx=dx, dg=dg)
    torch.cuda.synchronize()
    y_ref, dx_ref, dg_ref, dw_ref = oracle_all(inp, EPS)
    assert_acts_close("y", y, y_ref)
    assert_acts_close("dx", dx, dx_ref)
    assert_acts_close("dg", dg, dg_ref)
    assert_dw_close(dw, dw_ref, True)


def test_inplace_dx_rejected():
    inp = make_inputs(64, seed=13, device="cuda")
    with pytest.raises(binding.GatedRMSNormError, match="ALIAS"):
        binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], EPS,
                                  dx=inp["x"])


# --------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times.

def _sample_rows(rows, extra=None, seed=0):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(min(512, rows)),
                          np.arange(max(0, rows - 513), rows),
                          rng.integers(0, rows, 2048)])
    if extra is not None:
        idx = np.concatenate([idx, extra])
    return np.unique(idx)


@pytest.mark.parametrize("name", ["7684x48", "32768x48", "65536x48", "262144x48_outliers"])
def test_full_size_sampled(name):
    wl = WORKLOADS[name]
    say(f"[parity] {name} rows={wl.rows} full size, sampled rows")
    inp = make_workload_inputs(wl, device="cuda")
    y, dx, dg, dw32 = gpu_all(inp, wl.eps, True)
    extra = None
    if wl.outlier_frac > 0:
        big = (inp["x"].float().abs().amax(dim=1) > 20).nonzero().flatten()
        assert big.numel() >= int(wl.rows * wl.outlier_frac) * 0.99
        extra = big[:512].cpu().numpy()
    idx_np = _sample_rows(wl.rows, extra)
    idx = torch.from_numpy(idx_np).cuda()
    sub = {k: (v[idx] if k != "w" else v) for k, v in inp.items()}
    y_ref, dx_ref, dg_ref, _ = oracle_all(sub, wl.eps, want_dw=False)
    assert_acts_close("y", y[idx], y_ref)
    assert_acts_close("dx", dx[idx], dx_ref)
    assert_acts_close("dg", dg[idx], dg_ref)
    dw_ref = oracle_dw_streamed(inp, wl.eps)
    e32 = assert_dw_close(dw32, dw_ref, True)
    _, _, dw16 = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], wl.eps,
                                           dw_fp32=False)
    torch.cuda.synchronize()
    u16 = assert_dw_close(dw16, dw_ref, False)
    say(f"  dw fp32 rel err {e32:.2e}, dw bf16 worst {u16} ulp")


def test_tensors_beyond_4gib():
    """17,000,000 rows: each BF16 tensor is 4.35 GB, so byte offsets pass
    2^32 at row 16,777,216.  Rows on both sides of that boundary, sampled
    rows elsewhere and the whole dw (FP32 and BF16) against the oracle."""
    rows = 17_000_000
    say(f"[parity] rows={rows}: tensors beyond 4 GiB")
    inp = make_inputs(rows, seed=17, device="cuda")
    y, dx, dg, dw32 = gpu_all(inp, EPS, True)
    boundary = (1 << 32) // (128 * 2)
    idx_np = _sample_rows(rows, np.arange(boundary - 300, boundary + 300), seed=5)
    idx = torch.from_numpy(idx_np).cuda()
    sub = {k: (v[idx] if k != "w" else v) for k, v in inp.items()}
    y_ref, dx_ref, dg_ref, _ = oracle_all(sub, EPS, want_dw=False)
    assert_acts_close("y", y[idx], y_ref)
    assert_acts_close("dx", dx[idx], dx_ref)
    assert_acts_close("dg", dg[idx], dg_ref)
    del y, dx, dg
    dw_ref = oracle_dw_streamed(inp, EPS)
    e32 = assert_dw_close(dw32, dw_ref, True)
    _, _, dw16 = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], EPS,
                                           dw_fp32=False)
    torch.cuda.synchronize()
    u16 = assert_dw_close(dw16, dw_ref, False)
    say(f"  dw fp32 rel err {e32:.2e}, dw bf16 worst {u16} ulp")


# --------------------------------------------------------------------------
# Strided rows: x and g as the two halves of a fused projection, outputs
# into strided views.  Results must be bitwise those of packed copies.

def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


@pytest.mark.parametrize("rows,pitch", [(5000, 256), (1037, 136), (300, 1024), (1, 256)])
def test_strided_rows_match_packed(rows, pitch):
    say(f"[parity] strided rows={rows} pitch={pitch}")
    inp = make_inputs(rows, seed=31, device="cuda")
    proj = torch.full((rows, pitch * 2), float("nan"), dtype=torch.bfloat16, device="cuda")
    x = proj[:, :128]
    g = proj[:, pitch:pitch + 128]
    x.copy_(inp["x"])
    g.copy_(inp["g"])
    dy_buf = torch.full((rows, pitch), float("nan"), dtype=torch.bfloat16, device="cuda")
    dy = dy_buf[:, pitch - 128:]
    dy.copy_(inp["dy"])
    y_buf = torch.full((rows, pitch), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = y_buf[:, 8:136] if pitch >= 136 else y_buf[:, :128]
    dproj = torch.full((rows, pitch * 2), float("nan"), dtype=torch.bfloat16, device="cuda")
    dx = dproj[:, :128]
    dg = dproj[:, pitch:pitch + 128]
    keep_y = y_buf.clone()
    keep_d = dproj.clone()

    binding.gated_rmsnorm_fwd(x, g, inp["w"], EPS, y=y)
    _, _, dw = binding.gated_rmsnorm_bwd(x, g, inp["w"], dy, EPS, True, dx=dx, dg=dg)
    y_p = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], EPS)
    dx_p, dg_p, dw_p = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], EPS,
                                                 True)
    torch.cuda.synchronize()
    assert _bits_equal(y, y_p) and _bits_equal(dx, dx_p) and _bits_equal(dg, dg_p)
    assert torch.equal(dw.view(torch.int32), dw_p.view(torch.int32))
    # nothing outside the strided rows was written
    y_mask = torch.ones_like(y_buf, dtype=torch.bool)
    y_mask[:, 8:136] = False if pitch >= 136 else y_mask[:, 8:136]
    if pitch < 136:
        y_mask[:, :128] = False
    assert _bits_equal(y_buf[y_mask], keep_y[y_mask])
    d_mask = torch.ones_like(dproj, dtype=torch.bool)
    d_mask[:, :128] = False
    d_mask[:, pitch:pitch + 128] = False
    assert _bits_equal(dproj[d_mask], keep_d[d_mask])
    y_ref, dx_ref, dg_ref, dw_ref = oracle_all(inp, EPS)
    assert_acts_close("y", y, y_ref)
    assert_acts_close("dx", dx, dx_ref)
    assert_acts_close("dg", dg, dg_ref)
    assert_dw_close(dw, dw_ref, True)


def test_strided_ckpt_step_matches_packed():
    rows, pitch = 4099, 256
    say(f"[parity] strided ckpt rows={rows}")
    inp = make_inputs(rows, seed=32, device="cuda")
    proj = torch.empty((rows, 2 * pitch), dtype=torch.bfloat16, device="cuda")
    x, g = proj[:, :128], proj[:, pitch:pitch + 128]
    x.copy_(inp["x"])
    g.copy_(inp["g"])
    out = torch.empty((rows, 3 * pitch), dtype=torch.bfloat16, device="cuda")
    y, dx, dg = out[:, :128], out[:, pitch:pitch + 128], out[:, 2 * pitch:2 * pitch + 128]
    binding.gated_rmsnorm_ckpt_step(x, g, inp["w"], inp["dy"], EPS, False, y=y, dx=dx, dg=dg)
    ref = binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"], inp["dy"], EPS, False)
    torch.cuda.synchronize()
    for a, b in zip((y, dx, dg), ref[:3]):
        assert _bits_equal(a, b)

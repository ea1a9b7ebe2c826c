"""Run-to-run and launch-shape determinism on the GPU.

dw is summed in a fixed order that depends only on the number of rows, so
it must be bit-identical over repeated runs (with the workspace poisoned
between runs) and under any cap on the number of workgroups.  y, dx and dg
depend on their row only and must be bitwise stable too.  The checkpointed
step must give the same bits as fwd + bwd, and one workspace must serve
calls of any size (its counters return to zero).
"""
import os

import pytest
import torch

from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import WORKLOADS, make_inputs, make_workload_inputs

from gpu_util import say

pytestmark = pytest.mark.gpu


def _bwd_once(inp, eps, dw_fp32, ws):
    ws.fill_(float("nan"))                 # poison the scratch ...
    binding.gated_rmsnorm_workspace_init(ws)  # ... and zero the counters only
    dx, dg, dw = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], eps,
                                           dw_fp32=dw_fp32, workspace=ws)
    torch.cuda.synchronize()
    return dx, dg, dw


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("name", ["7684x48", "262144x48_outliers"])
def test_dw_bitwise_over_10_runs(name):
    wl = WORKLOADS[name]
    say(f"[determinism] {name} 10 runs")
    inp = make_workload_inputs(wl, device="cuda")
    ws = torch.empty(binding.gated_rmsnorm_workspace_bytes(wl.rows) // 4, device="cuda")
    modes = (True, False) if wl.rows < 10**6 else (True,)
    for dw_fp32 in modes:
        dx0, dg0, dw0 = _bwd_once(inp, wl.eps, dw_fp32, ws)
        dx0, dg0, dw0 = dx0.clone(), dg0.clone(), dw0.clone()
        for _ in range(9):
            dx, dg, dw = _bwd_once(inp, wl.eps, dw_fp32, ws)
            assert _same(dw, dw0)
            assert _same(dx, dx0) and _same(dg, dg0)


# 1,100,000 rows (282 MB per tensor) run the large-tensor backward, whose
# last-step stores are held back, with a ragged last chunk (96 rows).
@pytest.mark.parametrize("rows", [1100000, 368832, 49488, 1031, 257])
def test_launch_shape_invariance(rows, monkeypatch):
    say(f"[determinism] grid caps rows={rows}")
    inp = make_inputs(rows, seed=3, device="cuda")
    outs = []
    for cap in (None, "1", "7", "64"):
        if cap is None:
            monkeypatch.delenv("GATED_RMSNORM_MAX_WG", raising=False)
        else:
            monkeypatch.setenv("GATED_RMSNORM_MAX_WG", cap)
        y = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], 1e-6)
        dx, dg, dw = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"],
                                               1e-6, dw_fp32=True)
        torch.cuda.synchronize()
        outs.append((y, dx, dg, dw))
    monkeypatch.delenv("GATED_RMSNORM_MAX_WG", raising=False)
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert _same(a, b)


@pytest.mark.parametrize("dw_fp32", [True, False])
@pytest.mark.parametrize("rows", [9999, 200000])
def test_ckpt_step_equals_fwd_then_bwd(dw_fp32, rows):
    """9,999 rows run the recomputed forward inside the backward's launch
    (small tensors), 200,000 rows (49 MiB) as a launch of its own."""
    say(f"[determinism] ckpt vs fwd+bwd rows={rows} dw_fp32={dw_fp32}")
    inp = make_inputs(rows, seed=5, device="cuda")
    y1 = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], 1e-6)
    dx1, dg1, dw1 = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], 1e-6,
                                              dw_fp32=dw_fp32)
    y2, dx2, dg2, dw2 = binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"],
                                                        inp["dy"], 1e-6, dw_fp32=dw_fp32)
    torch.cuda.synchronize()
    for a, b in ((y1, y2), (dx1, dx2), (dg1, dg2), (dw1, dw2)):
        assert _same(a, b)


def test_ckpt_step_fused_with_tail_claims():
    """FP32 rows of D = 64 are 256 bytes: 131,071 rows stay below 32 MiB per
    tensor (the recomputed forward runs inside the backward's launch) and
    make 1,024 chunks (the backward claims its last 256 at run time), so one
    launch holds backward items, claim items, reducer items and forward
    tiles.  The step must equal fwd then bwd bit for bit, twice in a row on
    one workspace (the claim counter returns to zero)."""
    rows, D = 131071, 64
    say(f"[determinism] fused ckpt with tail claims rows={rows} D={D} FP32")
    inp = make_inputs(rows, D, seed=13, device="cuda", dtype=torch.float32)
    y1 = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], 1e-6)
    dx1, dg1, dw1 = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], 1e-6,
                                              dw_fp32=True)
    ws = binding.new_workspace(rows, "cuda", D=D)
    for _ in range(2):
        y2, dx2, dg2, dw2 = binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"],
                                                            inp["dy"], 1e-6, dw_fp32=True,
                                                            workspace=ws)
        torch.cuda.synchronize()
        for a, b in ((y1, y2), (dx1, dx2), (dg1, dg2), (dw1, dw2)):
            assert _same(a, b)
    C = binding.load_library().gated_rmsnorm_workspace_init_bytes()
    assert torch.count_nonzero(ws[:C]).item() == 0


def test_workspace_reused_across_sizes():
    """The counters return to zero after each call: one workspace serves
    calls of different sizes in any order, with the same bits as fresh ones.
    The sizes give 40, 5 and 115 groups, i.e. different spacings of the
    group counters (64, 64 and 32 words)."""
    sizes = (200000, 3001, 1700000)
    say(f"[determinism] workspace reuse rows={sizes}")
    inps = [make_inputs(r, seed=9 + k, device="cuda") for k, r in enumerate(sizes)]
    need = max(binding.gated_rmsnorm_workspace_bytes(r) for r in sizes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    order = (0, 1, 2, 0, 1, 1, 2, 2, 0)
    outs = []
    for k in order:
        inp = inps[k]
        outs.append(binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], 1e-6,
                                              dw_fp32=True, workspace=ws))
    torch.cuda.synchronize()
    fresh = [binding.gated_rmsnorm_bwd(i["x"], i["g"], i["w"], i["dy"], 1e-6, dw_fp32=True)
             for i in inps]
    torch.cuda.synchronize()
    for out, k in zip(outs, order):
        for x, y in zip(out, fresh[k]):
            assert _same(x, y)
    C = binding.load_library().gated_rmsnorm_workspace_init_bytes()
    assert torch.count_nonzero(ws[:C]).item() == 0


def test_nondefault_stream():
    rows = 3000
    say(f"[determinism] side stream rows={rows}")
    inp = make_inputs(rows, seed=8, device="cuda")
    ref = binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"], inp["dy"], 1e-6, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"], inp["dy"], 1e-6,
                                              True)
    s.synchronize()
    for a, b in zip(ref, out):
        assert _same(a, b)


def test_concurrent_streams():
    """Two backwards in flight at once on two streams (default priority),
    each with its own workspace, give the bits of the same calls made one
    after the other: the library keeps no state between calls."""
    rows_a, rows_b = 200000, 123457
    say(f"[determinism] concurrent streams rows={rows_a},{rows_b}")
    a = make_inputs(rows_a, seed=21, device="cuda")
    b = make_inputs(rows_b, seed=22, device="cuda")
    ref_a = binding.gated_rmsnorm_bwd(a["x"], a["g"], a["w"], a["dy"], 1e-6, dw_fp32=True)
    ref_b = binding.gated_rmsnorm_bwd(b["x"], b["g"], b["w"], b["dy"], 1e-6, dw_fp32=False)
    torch.cuda.synchronize()
    ws_a = binding.new_workspace(rows_a, "cuda")
    ws_b = binding.new_workspace(rows_b, "cuda")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a, outs_b = [], []
    for _ in range(3):
        with torch.cuda.stream(sa):
            outs_a.append(binding.gated_rmsnorm_bwd(a["x"], a["g"], a["w"], a["dy"], 1e-6,
                                                    dw_fp32=True, workspace=ws_a))
        with torch.cuda.stream(sb):
            outs_b.append(binding.gated_rmsnorm_bwd(b["x"], b["g"], b["w"], b["dy"], 1e-6,
                                                    dw_fp32=False, workspace=ws_b))
    torch.cuda.synchronize()
    for out in outs_a:
        for x, y in zip(out, ref_a):
            assert _same(x, y)
    for out in outs_b:
        for x, y in zip(out, ref_b):
            assert _same(x, y)


@pytest.mark.parametrize("rows", [600000, 4300000])
def test_forward_tile_size_invariance(rows):
    """The forward picks its tile and workgroup size by tensor size (16-row
    tiles from 128 MiB, 8-row tiles again from 1 GiB); a row's y must not
    depend on it: rows of a large call equal the same rows computed in a
    small call, bit for bit.  600,000 rows are 146 MiB per BF16 tensor,
    4,300,000 rows 1.03 GiB."""
    say(f"[determinism] forward tile size rows={rows}")
    inp = make_inputs(rows, seed=12, device="cuda")
    y_big = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], 1e-6)
    for lo, hi in ((0, 4099), (rows - 3001, rows), (250000, 260003)):
        y_small = binding.gated_rmsnorm_fwd(inp["x"][lo:hi].contiguous(),
                                            inp["g"][lo:hi].contiguous(), inp["w"], 1e-6)
        torch.cuda.synchronize()
        assert _same(y_big[lo:hi].contiguous(), y_small)

"""The checkpointed step (forward, recomputed forward, backward) against the
FP64 oracle.

flashinfer PR #8701, "How the tables were measured", defines the step as two
forwards and a backward captured in one graph (ckptg; stepg_f32 with an FP32
weight gradient).  Here the step's own outputs are compared with the oracle,
element by element, not only with this library's separate fwd and bwd:

* 1031x48 (49,488 rows, 12.7 MB per tensor) in full, both dw types: below
  32 MiB per tensor the recomputed forward runs inside the backward's launch.
  With GATED_RMSNORM_CKPT_SKIP_FIRST_FWD set, y starts as NaN and is written
  by those fused forward tiles alone, so they are checked directly; FP16 and
  FP32 storage reach their own fused instantiations.
* 65536x48 (3,145,728 rows, 805 MB per tensor) with an FP32 dw, as the
  largest-but-one workload states it: the step captured into one HIP graph on
  a zeroed workspace and replayed twice, with eager work between the
  replays.  y, dx and dg on sampled rows (both ends and 2,048 random rows),
  the whole dw against the oracle's streamed sum; the two replays agree bit
  for bit and leave the workspace's counters at zero.
"""
import numpy as np
import pytest
import torch

import oracle
from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import WORKLOADS, make_inputs, make_workload_inputs

from _compare import Y_TOL_F16, Y_TOL_F32, act_err, dw32_err, dwf16_check, DW32_TOL
from gpu_util import (assert_acts_close, assert_dw_close, bits, oracle_all, oracle_dw_streamed,
                      say)

pytestmark = pytest.mark.gpu
SKIP_FIRST = "GATED_RMSNORM_CKPT_SKIP_FIRST_FWD"


def _nan_like(t):
    return torch.full_like(t, float("nan"))


@pytest.mark.parametrize("skip_first", [False, True])
@pytest.mark.parametrize("dw_fp32", [False, True])
def test_ckpt_step_1031x48_full(dw_fp32, skip_first, monkeypatch):
    wl = WORKLOADS["1031x48"]
    say(f"[ckpt] {wl.name} rows={wl.rows} full, dw_fp32={dw_fp32}, "
        f"recomputed forward only={skip_first}")
    if skip_first:
        monkeypatch.setenv(SKIP_FIRST, "1")
    else:
        monkeypatch.delenv(SKIP_FIRST, raising=False)
    inp = make_workload_inputs(wl, device="cuda")
    y = _nan_like(inp["x"])
    dx = _nan_like(inp["x"])
    dg = _nan_like(inp["x"])
    dw = torch.full((128,), float("nan"), device="cuda",
                    dtype=torch.float32 if dw_fp32 else torch.bfloat16)
    binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"], inp["dy"], wl.eps,
                                    dw_fp32=dw_fp32, y=y, dx=dx, dg=dg, dw=dw)
    torch.cuda.synchronize()
    monkeypatch.delenv(SKIP_FIRST, raising=False)
    for t in (y, dx, dg):
        assert not torch.isnan(t).any().item()
    y_ref, dx_ref, dg_ref, dw_ref = oracle_all(inp, wl.eps)
    ey = assert_acts_close("y", y, y_ref)
    ex = assert_acts_close("dx", dx, dx_ref)
    eg = assert_acts_close("dg", dg, dg_ref)
    ew = assert_dw_close(dw, dw_ref, dw_fp32)
    say(f"  y {ey:.2e} dx {ex:.2e} dg {eg:.2e} dw {ew}")


@pytest.mark.parametrize("dname,D", [("f16", 128), ("f16", 256), ("f32", 64)])
def test_ckpt_fused_forward_other_types(dname, D, monkeypatch):
    """The fused forward tiles of FP16 and FP32 storage, alone (the first
    forward skipped), against the oracle."""
    dtype = {"f16": torch.float16, "f32": torch.float32}[dname]
    bar = {"f16": Y_TOL_F16, "f32": Y_TOL_F32}[dname]
    rows = 20011
    say(f"[ckpt] fused forward only {dname} D={D} rows={rows}")
    inp = make_inputs(rows, D, seed=41, device="cuda", dtype=dtype)
    y = _nan_like(inp["x"])
    monkeypatch.setenv(SKIP_FIRST, "1")
    _, dx, dg, dw = binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"], inp["dy"],
                                                    1e-6, dw_fp32=False, y=y)
    torch.cuda.synchronize()
    monkeypatch.delenv(SKIP_FIRST, raising=False)
    a = {k: np.ascontiguousarray(v.detach().cpu().double().numpy()) for k, v in inp.items()}
    y_ref = oracle.fwd(a["x"], a["g"], a["w"], 1e-6)
    dx_ref, dg_ref, dw_ref = oracle.bwd(a["x"], a["g"], a["w"], a["dy"], 1e-6)
    for name, t, r in (("y", y, y_ref), ("dx", dx, dx_ref), ("dg", dg, dg_ref)):
        err, _, _ = act_err(t.cpu().double().numpy(), r)
        assert err <= bar, f"{name}: rel err {err:.3e} > {bar:.0e}"
    if dtype == torch.float16:
        worst, ok = dwf16_check(dw.cpu().numpy().view(np.uint16), dw_ref)
        assert ok, f"dw off by {worst} ulp"
    else:
        assert dw32_err(dw.cpu().double().numpy(), dw_ref) <= DW32_TOL


def test_ckpt_step_65536x48_graph_fp32_dw():
    wl = WORKLOADS["65536x48"]
    rows = wl.rows
    say(f"[ckpt] {wl.name} rows={rows}: step captured in one graph, FP32 dw, 2 replays")
    inp = make_workload_inputs(wl, device="cuda")
    x, g, w, dy = inp["x"], inp["g"], inp["w"], inp["dy"]
    y, dx, dg = (torch.empty_like(x) for _ in range(3))
    dw = torch.empty(128, dtype=torch.float32, device="cuda")
    ws = binding.new_workspace(rows, "cuda")          # zero-filled
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        binding.gated_rmsnorm_ckpt_step(x, g, w, dy, wl.eps, dw_fp32=True, y=y, dx=dx, dg=dg,
                                        dw=dw, workspace=ws)
    torch.cuda.synchronize()
    outs = []
    for rep in range(2):
        for t in (y, dx, dg):
            t.fill_(float("nan"))
        dw.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        outs.append(tuple(t.clone() for t in (y, dx, dg, dw)))
        # eager work between the replays
        binding.gated_rmsnorm_fwd(x[:1000], g[:1000], w, wl.eps)
        torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
    C = binding.load_library().gated_rmsnorm_workspace_init_bytes()
    assert torch.count_nonzero(ws[:C]).item() == 0
    y, dx, dg, dw = outs[0]
    del outs
    rng = np.random.default_rng(65536)
    idx_np = np.unique(np.concatenate([np.arange(1024), np.arange(rows - 1024, rows),
                                       rng.integers(0, rows, 2048)]))
    idx = torch.from_numpy(idx_np).cuda()
    sub = {k: (v[idx] if k != "w" else v) for k, v in inp.items()}
    y_ref, dx_ref, dg_ref, _ = oracle_all(sub, wl.eps, want_dw=False)
    ey = assert_acts_close("y", y[idx], y_ref)
    ex = assert_acts_close("dx", dx[idx], dx_ref)
    eg = assert_acts_close("dg", dg[idx], dg_ref)
    del y, dx, dg
    dw_ref = oracle_dw_streamed(inp, wl.eps)
    ew = assert_dw_close(dw, dw_ref, True)
    say(f"  sampled rows {idx_np.size}: y {ey:.2e} dx {ex:.2e} dg {eg:.2e}; dw rel {ew:.2e}")

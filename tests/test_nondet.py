"""The non-deterministic dw option (``deterministic=False``).

dw is then summed with FP32 float atomics, one add per 128-row chunk, in
whatever order the chunks finish, so its bits may change from run to run;
the per-row outputs dx and dg come from the same code as the deterministic
path and must equal it bit for bit.  dw is held to the same oracle bars as
the deterministic dw (FP32 relative 1e-4, BF16 within 2 ulp).  The
accumulator and its counter live in the workspace's counter region and are
returned to zero by the call, so a workspace serves both options in turn.
"""
import pytest
import torch

from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import WORKLOADS, make_inputs, make_workload_inputs

from gpu_util import assert_dw_close, oracle_all, oracle_dw_streamed, say

pytestmark = pytest.mark.gpu


def _eq(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _both(inp, eps, dw_fp32, **kw):
    det = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], eps,
                                    dw_fp32=dw_fp32, **kw)
    nd = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], eps,
                                   dw_fp32=dw_fp32, deterministic=False, **kw)
    torch.cuda.synchronize()
    return det, nd


@pytest.mark.parametrize("rows", [1, 33, 129, 1031, 49488])
def test_nondet_small_against_oracle(rows):
    say(f"[nondet] rows={rows} vs oracle")
    inp = make_inputs(rows, seed=40 + rows % 7, device="cuda")
    _, _, _, dw_ref = oracle_all(inp, 1e-6)
    for dw_fp32 in (True, False):
        (dx, dg, _), (dx2, dg2, dw2) = _both(inp, 1e-6, dw_fp32)
        assert _eq(dx, dx2) and _eq(dg, dg2)
        assert_dw_close(dw2, dw_ref, dw_fp32)


@pytest.mark.parametrize("name", ["7684x48", "262144x48_outliers"])
def test_nondet_full_size(name):
    wl = WORKLOADS[name]
    say(f"[nondet] {name} rows={wl.rows} full size")
    inp = make_workload_inputs(wl, device="cuda")
    dw_ref = oracle_dw_streamed(inp, wl.eps)
    for dw_fp32 in (True, False):
        (dx, dg, _), (dx2, dg2, dw2) = _both(inp, wl.eps, dw_fp32)
        assert _eq(dx, dx2) and _eq(dg, dg2)
        e = assert_dw_close(dw2, dw_ref, dw_fp32)
        say(f"  dw_fp32={dw_fp32}: {e}")


def test_nondet_ckpt_step():
    rows = 9999
    say(f"[nondet] ckpt step rows={rows}")
    inp = make_inputs(rows, seed=44, device="cuda")
    _, _, _, dw_ref = oracle_all(inp, 1e-6)
    ref = binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"], inp["dy"], 1e-6, True)
    out = binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"], inp["dy"], 1e-6, True,
                                          deterministic=False)
    torch.cuda.synchronize()
    for a, b in zip(ref[:3], out[:3]):
        assert _eq(a, b)
    assert_dw_close(out[3], dw_ref, True)


@pytest.mark.parametrize("cap", [None, "1", "7"])
def test_nondet_leaves_workspace_clean(cap, monkeypatch):
    """After a non-deterministic call the counter region is zero again and a
    deterministic call on the same workspace gives the fresh bits."""
    rows = 30000
    say(f"[nondet] workspace clean rows={rows} cap={cap}")
    if cap is not None:
        monkeypatch.setenv("GATED_RMSNORM_MAX_WG", cap)
    inp = make_inputs(rows, seed=45, device="cuda")
    ws = binding.new_workspace(rows, "cuda")
    ws.fill_(0xFF)
    binding.gated_rmsnorm_workspace_init(ws)
    C = binding.load_library().gated_rmsnorm_workspace_init_bytes()
    _, _, _, dw_ref = oracle_all(inp, 1e-6)
    (dx, dg, dw), (dx2, dg2, dw2) = _both(inp, 1e-6, True, workspace=ws)
    assert torch.count_nonzero(ws[:C]).item() == 0
    assert _eq(dx, dx2) and _eq(dg, dg2)
    assert_dw_close(dw2, dw_ref, True)
    fresh = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], 1e-6, True)
    again = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], 1e-6, True,
                                      workspace=ws)
    torch.cuda.synchronize()
    assert _eq(dw, fresh[2]) and _eq(again[2], fresh[2])
    assert torch.count_nonzero(ws[:C]).item() == 0


def test_nondet_graph_replays():
    rows = 20000
    say(f"[nondet] graph replays rows={rows}")
    inp = make_inputs(rows, seed=46, device="cuda")
    x, g, w, dy = inp["x"], inp["g"], inp["w"], inp["dy"]
    _, _, _, dw_ref = oracle_all(inp, 1e-6)
    dx_e, dg_e, _ = binding.gated_rmsnorm_bwd(x, g, w, dy, 1e-6, dw_fp32=True)
    dx, dg = torch.empty_like(x), torch.empty_like(x)
    dw = torch.empty(128, dtype=torch.float32, device="cuda")
    ws = binding.new_workspace(rows, "cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.gated_rmsnorm_bwd(x, g, w, dy, 1e-6, True, dx=dx, dg=dg, dw=dw, workspace=ws,
                                  deterministic=False)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        binding.gated_rmsnorm_bwd(x, g, w, dy, 1e-6, True, dx=dx, dg=dg, dw=dw, workspace=ws,
                                  deterministic=False)
    for _ in range(4):
        dx.zero_(), dg.zero_(), dw.fill_(float("nan"))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert _eq(dx, dx_e) and _eq(dg, dg_e)
        assert_dw_close(dw, dw_ref, True)

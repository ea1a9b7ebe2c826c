"""HIP-graph capture of the C-ABI calls.

The library only enqueues kernels on the caller's stream (no allocation, no
synchronization, no memset), so fwd, bwd and the checkpointed step can be
captured.  Each graph is replayed several times with eager work and
synchronizations in between, and every replay must equal the eager result
bit for bit.  20,000 rows (5 MB per tensor) run the checkpointed step as two
launches (the recomputed forward inside the backward's) with 157 chunks;
200,000 rows (51 MB) run it as three launches, and their 1,563 chunks make
the backward hand out its last 256 chunks at run time through a counter that
every replay must leave at zero, with the other arrival counters.
"""
import pytest
import torch

from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import make_inputs

from gpu_util import say

pytestmark = pytest.mark.gpu


def _eq(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("dw_fp32", [True, False])
@pytest.mark.parametrize("rows", [20000, 200000])
def test_graph_replay_matches_eager(dw_fp32, rows):
    say(f"[graph] capture/replay rows={rows} dw_fp32={dw_fp32}")
    inp = make_inputs(rows, seed=21, device="cuda")
    x, g, w, dy = inp["x"], inp["g"], inp["w"], inp["dy"]
    dwt = torch.float32 if dw_fp32 else torch.bfloat16
    y_e = binding.gated_rmsnorm_fwd(x, g, w, 1e-6)
    dx_e, dg_e, dw_e = binding.gated_rmsnorm_bwd(x, g, w, dy, 1e-6, dw_fp32=dw_fp32)
    torch.cuda.synchronize()

    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    dg = torch.empty_like(x)
    dw = torch.empty(128, dtype=dwt, device="cuda")
    ws = binding.new_workspace(rows, "cuda")
    y2 = torch.empty_like(x)
    dx2 = torch.empty_like(x)
    dg2 = torch.empty_like(x)
    dw2 = torch.empty(128, dtype=dwt, device="cuda")

    g_fwd, g_bwd, g_ckpt = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        # one eager call on the capture stream first (device facts are cached)
        binding.gated_rmsnorm_fwd(x, g, w, 1e-6, y=y)
    torch.cuda.synchronize()
    with torch.cuda.graph(g_fwd, stream=s):
        binding.gated_rmsnorm_fwd(x, g, w, 1e-6, y=y)
    with torch.cuda.graph(g_bwd, stream=s):
        binding.gated_rmsnorm_bwd(x, g, w, dy, 1e-6, dw_fp32=dw_fp32, dx=dx, dg=dg, dw=dw,
                                  workspace=ws)
    with torch.cuda.graph(g_ckpt, stream=s):
        binding.gated_rmsnorm_ckpt_step(x, g, w, dy, 1e-6, dw_fp32=dw_fp32, y=y2, dx=dx2,
                                        dg=dg2, dw=dw2, workspace=ws)
    for rep in range(4):
        for t in (y, dx, dg, y2, dx2, dg2):
            t.fill_(float("nan"))
        dw.fill_(float("nan"))
        dw2.fill_(float("nan"))
        torch.cuda.synchronize()
        g_fwd.replay()
        g_bwd.replay()
        torch.cuda.synchronize()
        assert _eq(y, y_e) and _eq(dx, dx_e) and _eq(dg, dg_e) and _eq(dw, dw_e), rep
        g_ckpt.replay()
        torch.cuda.synchronize()
        assert _eq(y2, y_e) and _eq(dx2, dx_e) and _eq(dg2, dg_e) and _eq(dw2, dw_e), rep
        # eager work between replays
        binding.gated_rmsnorm_fwd(x, g, w, 1e-6)
        torch.cuda.synchronize()
    C = binding.load_library().gated_rmsnorm_workspace_init_bytes()
    assert torch.count_nonzero(ws[:C]).item() == 0

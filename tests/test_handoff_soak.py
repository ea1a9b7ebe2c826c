"""Soak of the backward's cross-workgroup dw hand-off.

Every chunk's FP32 partial is written by one workgroup and read by another
(the last to arrive at its group's counter), and the group sums the same way
once more; a wrong order between a partial's stores and the counter that
announces it would show up as a dw whose bits change from run to run.  Here
200 backwards at 7684x48 (368,832 rows, 2,882 chunks in 54 groups, the last
512 chunks handed out at run time) run on one workspace whose partials are
poisoned with NaN before every run (the arrival counters zeroed), alternating
BF16 and FP32 dw.  dx, dg and dw must equal the first run's bits every time;
the test stops at the first difference.
"""
import pytest
import torch

from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import WORKLOADS, make_workload_inputs

from gpu_util import say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_handoff_soak_200_runs():
    wl = WORKLOADS["7684x48"]
    say(f"[soak] {wl.name}: 200 backwards on one NaN-poisoned workspace")
    inp = make_workload_inputs(wl, device="cuda")
    x, g, w, dy = inp["x"], inp["g"], inp["w"], inp["dy"]
    ws = torch.empty(binding.gated_rmsnorm_workspace_bytes(wl.rows) // 4, device="cuda")
    dx, dg = torch.empty_like(x), torch.empty_like(x)
    dws = {True: torch.empty(128, dtype=torch.float32, device="cuda"),
           False: torch.empty(128, dtype=torch.bfloat16, device="cuda")}
    ref = {}
    for run in range(200):
        dw_fp32 = run % 2 == 0
        ws.fill_(float("nan"))
        binding.gated_rmsnorm_workspace_init(ws)
        binding.gated_rmsnorm_bwd(x, g, w, dy, wl.eps, dw_fp32=dw_fp32, dx=dx, dg=dg,
                                  dw=dws[dw_fp32], workspace=ws)
        torch.cuda.synchronize()
        if dw_fp32 not in ref:
            ref[dw_fp32] = (dx.clone(), dg.clone(), dws[dw_fp32].clone())
            continue
        rdx, rdg, rdw = ref[dw_fp32]
        assert torch.equal(_bits(dws[dw_fp32]), _bits(rdw)), f"dw differs at run {run}"
        assert torch.equal(_bits(dx), _bits(rdx)), f"dx differs at run {run}"
        assert torch.equal(_bits(dg), _bits(rdg)), f"dg differs at run {run}"

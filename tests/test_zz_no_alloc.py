"""The allocation-free backward (gated_rmsnorm_bwd_noalloc) against the
backward with a caller's workspace (gated_rmsnorm_bwd), through the C ABI.

Both run the same kernels, so their outputs must be the same bits.  Calls in
a row share the library's static scratch, whose arrival counters every
backward leaves at zero: a larger call, then a smaller one, then the larger
one again, with other dtypes and widths in between, and finally the call
captured into a HIP graph and replayed (the case it exists for).
"""
import ctypes

import pytest
import torch

from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import make_inputs

from gpu_util import assert_dw_close, assert_acts_close, oracle_all, say

pytestmark = pytest.mark.gpu
EPS = 1e-6
CODES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _noalloc(lib, inp, dw_fp32):
    x = inp["x"]
    dx, dg = torch.full_like(x, float("nan")), torch.full_like(x, float("nan"))
    dw = torch.full((x.shape[1],), float("nan"), device="cuda",
                    dtype=torch.float32 if dw_fp32 else x.dtype)
    st = lib.gated_rmsnorm_bwd_noalloc(
        x.data_ptr(), inp["g"].data_ptr(), inp["w"].data_ptr(), inp["dy"].data_ptr(),
        dx.data_ptr(), dg.data_ptr(), dw.data_ptr(), x.shape[0], x.shape[1], EPS,
        CODES[x.dtype], int(dw_fp32),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.gated_rmsnorm_status_string(st)
    return dx, dg, dw


def _with_workspace(inp, dw_fp32):
    return binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], EPS,
                                     dw_fp32=dw_fp32)


@pytest.mark.parametrize("order", ["large-small-large"])
def test_noalloc_matches_workspace_backward(order):
    lib = binding.load_library()
    cases = [(368832, 128, torch.bfloat16, False),   # 7684x48, BF16 dw
             (49488, 128, torch.bfloat16, True),     # 1031x48, FP32 dw (smaller)
             (20011, 256, torch.float16, False),
             (3001, 64, torch.float32, True),
             (368832, 128, torch.bfloat16, True)]    # the large one again
    for rows, D, dtype, dw_fp32 in cases:
        say(f"[noalloc] rows={rows} D={D} {dtype} dw_fp32={dw_fp32}")
        inp = make_inputs(rows, D, seed=rows % 1000, device="cuda", dtype=dtype)
        got = _noalloc(lib, inp, dw_fp32)
        ref = _with_workspace(inp, dw_fp32)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(_bits(a), _bits(b))
        if rows == 49488:
            _, dx_ref, dg_ref, dw_ref = oracle_all(inp, EPS)
            assert_acts_close("dx", got[0], dx_ref)
            assert_acts_close("dg", got[1], dg_ref)
            assert_dw_close(got[2], dw_ref, dw_fp32)


def test_noalloc_in_a_graph():
    lib = binding.load_library()
    rows = 200000
    say(f"[noalloc] graph capture rows={rows}")
    inp = make_inputs(rows, 128, seed=77, device="cuda")
    ref = _with_workspace(inp, True)
    x = inp["x"]
    dx, dg = torch.empty_like(x), torch.empty_like(x)
    dw = torch.empty(128, dtype=torch.float32, device="cuda")
    args = lambda: (x.data_ptr(), inp["g"].data_ptr(), inp["w"].data_ptr(),  # noqa: E731
                    inp["dy"].data_ptr(), dx.data_ptr(), dg.data_ptr(), dw.data_ptr(), rows,
                    128, EPS, 0, 1,
                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        assert lib.gated_rmsnorm_bwd_noalloc(*args()) == 0   # set up before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        assert lib.gated_rmsnorm_bwd_noalloc(*args()) == 0
    for rep in range(3):
        for t in (dx, dg, dw):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((dx, dg, dw), ref):
            assert torch.equal(_bits(a), _bits(b)), rep
        # eager work between replays, including an eager call on the scratch
        _noalloc(lib, make_inputs(1000, 128, seed=rep, device="cuda"), False)
        torch.cuda.synchronize()

"""Concurrent calls from several host threads, each on a stream of its own with
its own outputs and workspace (the header's threading rule): every result
must be bitwise the result of the same call made alone, since nothing the
calls share (the inputs, w, the library) is written.  Python releases the GIL
inside ctypes calls, so the enqueues of different threads really interleave;
each thread repeats its calls so that their kernels overlap on the device."""
import threading

import pytest
import torch

from silu_gated_rmsnorm_amd import binding
from silu_gated_rmsnorm_amd.inputs import make_inputs

from gpu_util import say

pytestmark = pytest.mark.gpu

EPS = 1e-6
REPEATS = 3

# rows, D, dtype, dw_fp32: sizes that take different kernel shapes (small tier
# with the fused checkpointed step; middle shape with tail claims; FP16 at
# D = 256; FP32 at D = 64 with claim, reducer and forward items in one launch).
CASES = [
    (49488, 128, torch.bfloat16, False),
    (368832, 128, torch.bfloat16, True),
    (20011, 256, torch.float16, False),
    (131071, 64, torch.float32, True),
]


def _calls(inp, dw_fp32, ws):
    y = binding.gated_rmsnorm_fwd(inp["x"], inp["g"], inp["w"], EPS)
    dx, dg, dw = binding.gated_rmsnorm_bwd(inp["x"], inp["g"], inp["w"], inp["dy"], EPS,
                                           dw_fp32=dw_fp32, workspace=ws)
    yc, dxc, dgc, dwc = binding.gated_rmsnorm_ckpt_step(inp["x"], inp["g"], inp["w"],
                                                        inp["dy"], EPS, dw_fp32=dw_fp32,
                                                        workspace=ws)
    return {"y": y, "dx": dx, "dg": dg, "dw": dw,
            "ckpt.y": yc, "ckpt.dx": dxc, "ckpt.dg": dgc, "ckpt.dw": dwc}


def _bytes(t):
    return t.contiguous().view(torch.uint8)


def test_concurrent_threads_match_serial_calls():
    dev = torch.device("cuda:0")
    inputs, refs = [], []
    for k, (rows, D, dt, dw_fp32) in enumerate(CASES):
        say(f"[threads] serial reference {rows}x{D} {dt} dw_fp32={dw_fp32}")
        inp = make_inputs(rows, D, seed=500 + k, device=dev, dtype=dt)
        ws = binding.new_workspace(rows, dev, D)
        out = _calls(inp, dw_fp32, ws)
        torch.cuda.synchronize()
        inputs.append(inp)
        refs.append({n: t.clone() for n, t in out.items()})
    torch.cuda.synchronize()

    start = threading.Barrier(len(CASES))
    failures = []

    def worker(k):
        rows, D, _, dw_fp32 = CASES[k]
        try:
            stream = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(stream):
                ws = binding.new_workspace(rows, dev, D)
                start.wait()
                for rep in range(REPEATS):
                    out = _calls(inputs[k], dw_fp32, ws)
                    stream.synchronize()
                    for name, t in out.items():
                        if not torch.equal(_bytes(t), _bytes(refs[k][name])):
                            failures.append(f"case {k} ({rows}x{D}) repeat {rep}: {name} differs")
                            return
        except Exception as e:  # reported by the main thread
            failures.append(f"case {k}: {type(e).__name__}: {e}")

    say(f"[threads] {len(CASES)} threads x {REPEATS} repeats")
    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(CASES))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=90)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not failures, "; ".join(failures)

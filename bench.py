#!/usr/bin/env python3
"""Benchmark of the SiLU-gated RMSNorm training forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 7684x48]
                    [--dtype bf16|f16|f32] [--dim 64|128|256]

A step is one training forward and backward over the workload: the forward
(y from x, g, w) followed by the backward (dx, dg and the deterministic BF16
dw, one kernel).  Set-up ends with untimed steps over every buffer set for
at least 50 ms (so that the GPU's clocks have settled and every buffer has
been touched); then W untimed warm-up steps run, then exactly K steps are
timed with HIP events on the stream the kernels are launched on, bracketed
by device synchronizations.  Inputs are synthetic (seeded) and resident in
HBM when timing starts.

Every timed loop rotates over several identical buffer sets (inputs copied,
outputs and workspace separate) that together span at least 1 GiB per
tensor role, four times the 256 MB Infinity Cache: a launch never finds its
inputs left in a cache by the previous launch, so the figures are HBM
figures.  Within one step the backward may still find part of x and g that
its forward just read; that reuse is the step's own.

stdout gets one JSON line; everything else goes to stderr.  Besides the step
throughput (an effective bandwidth: the step's algorithmic bytes over its
time) the line carries:
  * fwd_plus_bwd_apart: the same bytes over the forward and the backward
    timed apart (no reuse of x and g between them);
  * ops: per-operation timings at 7684x48: eager launches back to back, and
    the pages' graph operations (fwdg, bwdg, bwdg_f32, ckptg, stepg_f32) as
    GPU time per operation from N operations captured in one graph, with
    the wall time of one-operation graph replays as *_replay_wall;
  * roofline: the dominant kernel (the backward) against MI355X's 8 TB/s;
  * workloads: 1031x48, 32768x48, 65536x48 and 262144x48 with outlier rows,
    each in the operation it is quoted on, with the oracle timed beside it;
  * cpu_baseline: the FP64 CPU oracle on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
D = 128
ROW_BYTES = D * 2               # one BF16 row
ROTATION_BYTES = 1 << 30        # per tensor role, across the buffer sets
SETTLE_S = 0.05                 # untimed steps before the warm-up, seconds

# The pages' own timings of the same operations at T x H = 7684 x 48 on an
# NVIDIA R200 (sm_107a, 212 SMs, CUDA 13.4): flashinfer PR #8701, Table 2
# ("new us" and the deterministic package's column).  Context only.
R200_7684x48_US = {
    "fwd": 30.672, "fwdg": 30.553, "bwdg": 59.872, "bwdg_f32": 59.744,
    "ckptg": 118.449, "stepg_f32": 118.537, "fwd+bwd": 90.424,
    "det_fwd": 34.641, "det_bwdg": 65.896, "det_ckptg": 132.328,
}

PROFILES_DIR = ROOT / "profiles"


def counters_file(workload):
    """Committed HBM-traffic figures of the kernels for one workload."""
    return PROFILES_DIR / f"bwd_kernel_{workload}_traffic.json"

# The deterministic backward kernel (template arguments: element type, D, row
# groups per wave step, waves per workgroup, rows per chunk, prefetched
# steps, deterministic, last step's stores held back, fence per work item,
# window of chunks whose blocks interleave: 0 for the prefetching shape,
# recomputed forward fused in: only in the small checkpointed step).
BWD_KERNEL = ("grn::bwd_kernel<(grn::Dt){code}, {D}, {U}, 4, {R}, {PF}, true, {HOLD}, false, "
              "{SWZ}, false>")
# The sources the kernels are compiled from: the committed HBM counter
# figures apply only while their combined SHA-256 is the one recorded.
KERNEL_SOURCES = tuple(ROOT / "silu_gated_rmsnorm_amd" / "csrc" / name
                       for name in ("kernels.hip", "common.h", "launch.h"))


def kernel_source_sha():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        h.update(path.read_bytes())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="7684x48")
    p.add_argument("--settle-ms", type=float, default=SETTLE_S * 1e3,
                   help="untimed steps over every buffer set before the warm-up, in ms")
    p.add_argument("--dtype", choices=("bf16", "f16", "f32"), default="bf16",
                   help="storage type of x, g, dy, w and the outputs (the pages: bf16)")
    p.add_argument("--dim", type=int, choices=(64, 128, 256), default=D,
                   help="row width D (the pages: 128)")
    p.add_argument("--layout", choices=("packed", "fused"), default="packed",
                   help="packed rows, or x|g and dx|dg as the two halves of fused "
                        "[rows, 2D] buffers (row stride 2D)")
    p.add_argument("--op-reps", type=int, default=50,
                   help="launches per operation in the per-op timings")
    p.add_argument("--no-ops", action="store_true", help="skip per-op timings")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the other workloads (1031x48, 32768x48, 65536x48, "
                        "262144x48_outliers), timed by default beside 7684x48")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time of the oracle baseline")
    p.add_argument("--profile-op", choices=("fwd", "bwd", "ckpt"),
                   help="profiling mode: run only this operation (warmup, then "
                        "--op-reps launches in buffer rotation) and print its timing; "
                        "the profiler's per-kernel average then covers exactly these "
                        "launches")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files "
                        "(FETCH_SIZE, WRITE_SIZE) of this benchmark into the per-launch "
                        "HBM traffic summary under profiles/")
    return p.parse_args()


class Workbench:
    """One workload's buffer sets on the GPU and the raw C-ABI calls on them.

    Buffer sets are identical copies (inputs cloned, outputs and workspace
    separate) that together span at least ROTATION_BYTES per tensor role, so
    a launch that takes the next set never finds its inputs left in a cache
    by the launch before it."""

    def __init__(self, torch, binding, wl, D, tdtype, dt_code, layout, dev):
        from silu_gated_rmsnorm_amd.inputs import make_inputs

        self.torch, self.lib = torch, binding.load_library()
        self.wl, self.D, self.dt_code = wl, D, dt_code
        self.rows, self.eps = wl.rows, wl.eps
        esize = 4 if tdtype == torch.float32 else 2
        self.row_bytes = D * esize
        self.tensor_bytes = self.rows * self.row_bytes
        self.nsets = math.ceil(ROTATION_BYTES / self.tensor_bytes) + 1
        self.fused = layout == "fused"
        self.inp = make_inputs(self.rows, D, seed=0, device=dev, g_std=wl.g_std,
                               outlier_frac=wl.outlier_frac,
                               outlier_scale=wl.outlier_scale, dtype=tdtype)
        inp = self.inp
        self.ws_bytes = binding.gated_rmsnorm_workspace_bytes(self.rows, D)
        self.sets = []
        for _ in range(self.nsets):
            if self.fused:
                proj = torch.cat([inp["x"], inp["g"]], dim=1)
                dproj = torch.empty_like(proj)
                st = {"x": proj[:, :D], "g": proj[:, D:], "dy": inp["dy"].clone(),
                      "dx": dproj[:, :D], "dg": dproj[:, D:], "y": torch.empty_like(inp["x"])}
            else:
                st = {k: inp[k].clone() for k in ("x", "g", "dy")}
                for k in ("y", "dx", "dg"):
                    st[k] = torch.empty_like(inp["x"])
            st["w"] = inp["w"]
            st["dw16"] = torch.empty(D, dtype=tdtype, device=dev)   # dw in the input type
            st["dw32"] = torch.empty(D, dtype=torch.float32, device=dev)
            st["ws"] = binding.new_workspace(self.rows, dev, D)
            self.sets.append(st)
        torch.cuda.synchronize()
        # Algorithmic bytes: what the method must move (inputs read once,
        # outputs written once, w and dw included; workspace traffic, ~0.7 %
        # of the backward's, is implementation overhead and not counted).
        rb, rows = self.row_bytes, self.rows
        self.fwd_bytes = rows * 3 * rb + rb
        self.bwd_bytes = rows * 5 * rb + rb + D * esize
        self.bwd32_bytes = rows * 5 * rb + rb + D * 4
        self.ckpt_bytes = 2 * self.fwd_bytes + self.bwd_bytes
        self.ckpt32_bytes = 2 * self.fwd_bytes + self.bwd32_bytes
        self.step_bytes = self.fwd_bytes + self.bwd_bytes
        self.step32_bytes = self.fwd_bytes + self.bwd32_bytes

    # -- raw C-ABI calls on buffer set `st` (no per-call Python checks) -----
    def _s(self):
        return self.torch.cuda.current_stream().cuda_stream

    def _check(self, status):
        if status != 0:
            raise RuntimeError(self.lib.gated_rmsnorm_status_string(status).decode())

    def op_fwd(self, st):
        P, R_, lib = (lambda t: t.data_ptr()), (lambda t: t.stride(0)), self.lib
        if self.fused:
            self._check(lib.gated_rmsnorm_fwd_strided(
                P(st["x"]), R_(st["x"]), P(st["g"]), R_(st["g"]), P(st["w"]), P(st["y"]),
                R_(st["y"]), self.rows, self.D, self.eps, self.dt_code, self._s()))
        else:
            self._check(lib.gated_rmsnorm_fwd(P(st["x"]), P(st["g"]), P(st["w"]), P(st["y"]),
                                              self.rows, self.D, self.eps, self.dt_code,
                                              self._s()))

    def op_bwd(self, st, fp32=False, det=True):
        P, R_, lib = (lambda t: t.data_ptr()), (lambda t: t.stride(0)), self.lib
        dw = st["dw32"] if fp32 else st["dw16"]
        if self.fused or not det:
            self._check(lib.gated_rmsnorm_bwd_strided(
                P(st["x"]), R_(st["x"]), P(st["g"]), R_(st["g"]), P(st["w"]), P(st["dy"]),
                R_(st["dy"]), P(st["dx"]), R_(st["dx"]), P(st["dg"]), R_(st["dg"]), P(dw),
                P(st["ws"]), self.ws_bytes, self.rows, self.D, self.eps, self.dt_code,
                int(fp32), int(det), self._s()))
        else:
            self._check(lib.gated_rmsnorm_bwd(
                P(st["x"]), P(st["g"]), P(st["w"]), P(st["dy"]), P(st["dx"]), P(st["dg"]),
                P(dw), P(st["ws"]), self.ws_bytes, self.rows, self.D, self.eps, self.dt_code,
                int(fp32), self._s()))

    def op_ckpt(self, st, fp32=False):
        P, R_, lib = (lambda t: t.data_ptr()), (lambda t: t.stride(0)), self.lib
        dw = st["dw32"] if fp32 else st["dw16"]
        if self.fused:
            self._check(lib.gated_rmsnorm_ckpt_step_strided(
                P(st["x"]), R_(st["x"]), P(st["g"]), R_(st["g"]), P(st["w"]), P(st["dy"]),
                R_(st["dy"]), P(st["y"]), R_(st["y"]), P(st["dx"]), R_(st["dx"]), P(st["dg"]),
                R_(st["dg"]), P(dw), P(st["ws"]), self.ws_bytes, self.rows, self.D, self.eps,
                self.dt_code, int(fp32), 1, self._s()))
        else:
            self._check(lib.gated_rmsnorm_ckpt_step(
                P(st["x"]), P(st["g"]), P(st["w"]), P(st["dy"]), P(st["y"]), P(st["dx"]),
                P(st["dg"]), P(dw), P(st["ws"]), self.ws_bytes, self.rows, self.D, self.eps,
                self.dt_code, int(fp32), self._s()))

    def op_step(self, st, fp32=False):
        self.op_fwd(st)
        self.op_bwd(st, fp32)

    # -- timing -------------------------------------------------------------
    def rotate_time(self, fn, reps):
        """Average us per call over `reps` back-to-back eager calls, rotating
        sets, timed with HIP events on the stream the kernels run on."""
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            fn(self.sets[i % self.nsets])
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    def settle(self, fn, seconds):
        """Untimed set-up: run fn over every buffer set, pass after pass, for
        at least `seconds`, so that no timed launch is the first to touch its
        buffers and the GPU has left its idle clocks (with only 10 warm-up
        steps the first timed steps at 7684x48 ran 3 % slow)."""
        t0 = time.perf_counter()
        while True:
            for st in self.sets:
                fn(st)
            self.torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                break

    def graph_time(self, fn, n):
        """GPU time per operation: n operations (rotating over the sets)
        captured into one HIP graph; after one untimed replay, the median of
        three timed replays.  The host's launch and submission costs drop out
        and the launches run back to back.
        This is the figure comparable to the pages' graph timings (kernel
        time of ops replayed from a graph)."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s):
            for i in range(n):
                fn(self.sets[i % self.nsets])
        gr.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            gr.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / n)
        del gr
        return sorted(times)[1]

    def replay_wall(self, fn, reps):
        """Wall time per replay of a graph that holds one operation (one graph
        per buffer set, replayed in rotation): the GPU time of the operation
        plus one submission per replay."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graphs = []
        for st in self.sets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=s):
                fn(st)
            graphs.append(gr)
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
        by_set = {id(st): gr for st, gr in zip(self.sets, graphs)}
        us = self.rotate_time(lambda st: by_set[id(st)].replay(), reps)
        del graphs, by_set
        return us

    def free(self):
        self.sets.clear()
        self.inp = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def rate(us, nbytes):
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 3), "GB/s": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}


# The other workloads of the pages' T x 48 family, each timed in the
# operation it is quoted on (D = 128, BF16, eps = 1e-6, seed 0):
#   1031x48: the forward and the backward with a BF16 dw;
#   32768x48: the forward and the backward timed apart, and their sum;
#   65536x48: the checkpointed step (2 x forward + backward) with an FP32 dw,
#             captured in one HIP graph;
#   262144x48 with 1 % outlier rows (x100) and g of standard deviation 2:
#             forward + backward with an FP32 dw, and dw bitwise over 10 runs.
# GPU figures are GPU time per operation from N operations captured in one
# graph (buffers rotated); the oracle is timed beside each (median of 3
# passes for the first two, one pass in 1 M-row chunks for the last two).
SIDE_WORKLOADS = ("1031x48", "32768x48", "65536x48", "262144x48_outliers")


def side_workload(torch, binding, name, dev, settle_s):
    from silu_gated_rmsnorm_amd.inputs import WORKLOADS

    wl = WORKLOADS[name]
    wb = Workbench(torch, binding, wl, 128, torch.bfloat16, 0, "packed", dev)
    log(f"[bench] workload {name}: rows={wl.rows} buffer sets={wb.nsets}")
    out = {"rows": wl.rows, "D": 128, "io_dtype": "bf16", "buffer_sets": wb.nsets,
           "timing": "GPU time per operation: N operations captured in one HIP graph, "
                     "buffer sets rotated"}
    ops = {}
    n = max(2 * wb.nsets, 100)
    if name == "1031x48":
        wb.settle(lambda st: wb.op_step(st), settle_s)
        ops["fwd"] = rate(wb.graph_time(wb.op_fwd, n), wb.fwd_bytes)
        ops["bwd"] = rate(wb.graph_time(wb.op_bwd, n), wb.bwd_bytes)
        ops["fwd+bwd"] = rate(ops["fwd"]["us"] + ops["bwd"]["us"], wb.step_bytes)
        cpu = cpu_oracle(wl, wb.inp, ("fwd", "bwd"), wb.step_bytes, repeats=3)
    elif name == "32768x48":
        wb.settle(lambda st: wb.op_step(st), settle_s)
        ops["fwd"] = rate(wb.graph_time(wb.op_fwd, n), wb.fwd_bytes)
        ops["bwd"] = rate(wb.graph_time(wb.op_bwd, n), wb.bwd_bytes)
        ops["fwd+bwd"] = rate(ops["fwd"]["us"] + ops["bwd"]["us"], wb.step_bytes)
        cpu = cpu_oracle(wl, wb.inp, ("fwd", "bwd"), wb.step_bytes, repeats=3)
    elif name == "65536x48":
        step = lambda st: wb.op_ckpt(st, True)  # noqa: E731
        wb.settle(step, settle_s)
        ops["stepg_f32"] = rate(wb.graph_time(step, n), wb.ckpt32_bytes)
        ops["stepg_f32_replay_wall"] = rate(wb.replay_wall(step, 2 * wb.nsets),
                                            wb.ckpt32_bytes)
        cpu = cpu_oracle(wl, wb.inp, ("fwd", "fwd", "bwd"), wb.ckpt32_bytes, repeats=1)
    else:
        step = lambda st: wb.op_step(st, True)  # noqa: E731
        wb.settle(step, settle_s)
        ops["fwd+bwd_f32"] = rate(wb.graph_time(step, n), wb.step32_bytes)
        ops["fwd+bwd_f32_eager"] = rate(wb.rotate_time(step, n), wb.step32_bytes)
        st = wb.sets[0]
        dws = []
        for _ in range(10):
            wb.op_bwd(st, True)
            torch.cuda.synchronize()
            dws.append(st["dw32"].clone())
        out["dw_bitwise_10_runs"] = all(torch.equal(d.view(torch.int32), dws[0].view(torch.int32))
                                        for d in dws)
        cpu = cpu_oracle(wl, wb.inp, ("fwd", "bwd"), wb.step32_bytes, repeats=1)
    for k, v in ops.items():
        log(f"[bench]   {name:20s} {k:24s} {v['us']:10.2f} us {v['GB/s']:8.1f} GB/s "
            f"{100 * v['frac']:5.1f}%")
    out["ops"] = ops
    out["cpu_baseline"] = cpu
    wb.free()
    return out


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, workload=args.workload)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this operator's hot path is measured on a "
              "single MI355X (rows are independent; sharding across GPUs is a design "
              "note, not part of this build). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")

    import torch

    from silu_gated_rmsnorm_amd import binding
    from silu_gated_rmsnorm_amd.inputs import WORKLOADS

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    wl = WORKLOADS[args.workload]
    rows, eps = wl.rows, wl.eps
    D = args.dim
    tdtype = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[args.dtype]
    dt_code = {"bf16": 0, "f16": 1, "f32": 2}[args.dtype]
    row_bytes = D * (4 if args.dtype == "f32" else 2)
    default_shape = (args.dtype, D, args.layout) == ("bf16", 128, "packed")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wb = Workbench(torch, binding, wl, D, tdtype, dt_code, args.layout, dev)
    nsets, settle_s = wb.nsets, args.settle_ms * 1e-3
    log(f"[bench] workload {wl.name}: rows={rows} D={D} dtype={args.dtype} eps={eps} "
        f"buffer sets={nsets} lib={binding.library_path()}")

    if args.profile_op:
        fn, nbytes = {"fwd": (wb.op_fwd, wb.fwd_bytes), "bwd": (wb.op_bwd, wb.bwd_bytes),
                      "ckpt": (wb.op_ckpt, wb.ckpt_bytes)}[args.profile_op]
        wb.settle(fn, settle_s)
        for i in range(args.warmup):
            fn(wb.sets[i % nsets])
        us = wb.rotate_time(fn, args.op_reps)
        gbps = nbytes / (us * 1e-6) / 1e9
        print(json.dumps({"profile_op": args.profile_op, "workload": wl.name,
                          "layout": args.layout, "dtype": args.dtype, "D": D,
                          "launches": args.op_reps, "avg_us_events": round(us, 3),
                          "GB/s": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}),
              flush=True)
        return

    # ---- the contract measurement: K timed steps --------------------------
    wb.settle(wb.op_step, settle_s)
    for i in range(args.warmup):
        wb.op_step(wb.sets[i % nsets])
    torch.cuda.synchronize()
    step_us = wb.rotate_time(wb.op_step, args.steps)
    ms_per_step = step_us / 1e3
    value = wb.step_bytes / (step_us * 1e-6) / 1e9
    log(f"[bench] step (fwd + bwd, {args.dtype} dw): {step_us:.2f} us, {value:.1f} GB/s "
        f"effective ({100 * value / HBM_PEAK_GBPS:.1f}% of 8 TB/s)")

    ops = {}
    roofline = None
    apart = None
    runtime_copy = None
    if not args.no_ops:
        R = args.op_reps

        def rec(name, r):
            ops[name] = r
            log(f"[bench] {name:24s} {r['us']:9.2f} us {r['GB/s']:8.1f} GB/s "
                f"{100 * r['frac']:5.1f}%")

        for st in wb.sets:
            wb.op_ckpt(st)
        torch.cuda.synchronize()
        # Eager launches, back to back, rotating sets.
        rec("fwd", rate(wb.rotate_time(wb.op_fwd, R), wb.fwd_bytes))
        bwd_us = wb.rotate_time(wb.op_bwd, R)
        rec("bwd", rate(bwd_us, wb.bwd_bytes))
        rec("bwd_f32", rate(wb.rotate_time(lambda st: wb.op_bwd(st, True), R), wb.bwd32_bytes))
        # A/B: dw summed with FP64 atomics instead of the fixed-order tree.
        rec("bwd_nondet", rate(wb.rotate_time(lambda st: wb.op_bwd(st, False, False), R),
                               wb.bwd_bytes))
        rec("bwd_nondet_f32", rate(wb.rotate_time(lambda st: wb.op_bwd(st, True, False), R),
                                   wb.bwd32_bytes))
        rec("ckpt", rate(wb.rotate_time(wb.op_ckpt, R), wb.ckpt_bytes))
        rec("ckpt_f32", rate(wb.rotate_time(lambda st: wb.op_ckpt(st, True), R),
                             wb.ckpt32_bytes))
        rec("fwd+bwd", rate(step_us, wb.step_bytes))
        rec("fwd+bwd_f32", rate(wb.rotate_time(lambda st: wb.op_step(st, True), R),
                                wb.step32_bytes))
        # The step's bytes over the two operations timed apart: no reuse of x
        # and g between the forward and the backward, an HBM-honest figure
        # beside the step's effective one.
        apart = rate(ops["fwd"]["us"] + ops["bwd"]["us"], wb.step_bytes)

        # The pages' graph operations (flashinfer PR #8701, "How the tables
        # were measured": fwdg, bwdg, bwdg_f32, ckptg, stepg_f32 are kernel
        # times of operations replayed from a graph): here GPU time per
        # operation from N operations captured in one graph.  Wall time per
        # replay of a one-operation graph (one submission each) is reported
        # as *_replay_wall.
        nb = max(2 * nsets, 100)
        kinds = {"fwdg": (wb.op_fwd, wb.fwd_bytes), "bwdg": (wb.op_bwd, wb.bwd_bytes),
                 "bwdg_f32": (lambda st: wb.op_bwd(st, True), wb.bwd32_bytes),
                 "bwdg_nondet": (lambda st: wb.op_bwd(st, False, False), wb.bwd_bytes),
                 "ckptg": (wb.op_ckpt, wb.ckpt_bytes),
                 "stepg_f32": (lambda st: wb.op_ckpt(st, True), wb.ckpt32_bytes),
                 "fwd+bwd_g": (wb.op_step, wb.step_bytes)}
        for name, (fn, nbytes) in kinds.items():
            rec(name, rate(wb.graph_time(fn, nb), nbytes))
        for name, (fn, nbytes) in kinds.items():
            rec(name + "_replay_wall", rate(wb.replay_wall(fn, R), nbytes))
        rec("fwdg+bwdg", rate(ops["fwdg"]["us"] + ops["bwdg"]["us"], wb.step_bytes))

        # Same buffers every launch (no rotation): inputs partly served by the
        # Infinity Cache; reported for contrast only.
        one = wb.sets[0]
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        for name, fn, nbytes in (("fwd_same_buffers", wb.op_fwd, wb.fwd_bytes),
                                 ("bwd_same_buffers", wb.op_bwd, wb.bwd_bytes)):
            fn(one)
            torch.cuda.synchronize()
            a.record()
            for _ in range(R):
                fn(one)
            b.record()
            torch.cuda.synchronize()
            rec(name, rate(a.elapsed_time(b) * 1e3 / R, nbytes))

        # Roofline of the dominant kernel: the backward is one kernel launch
        # (rows > 0), timed over back-to-back launches on its stream.
        achieved = wb.bwd_bytes / (bwd_us * 1e-6) / 1e9
        # The library picks the backward's shape by tensor size (32 MiB and
        # 256 MiB boundaries), and above 256 MiB by type and width: row
        # groups per wave step, prefetched steps, held stores and the window
        # of interleaved chunks.
        tb = rows * row_bytes
        prefetch = tb >= (256 << 20) and ((args.dtype == "f16" and D <= 128) or
                                          (args.dtype == "bf16" and D == 64))
        u, pf = (2, 1) if tb < (32 << 20) else ((4, 1) if prefetch else (4, 0))
        hold = prefetch and args.dtype == "bf16"
        kname = BWD_KERNEL.format(code=dt_code, D=D, U=u, R=256 if row_bytes <= 128 else 128,
                                  PF=pf, HOLD="true" if hold else "false",
                                  SWZ=0 if prefetch else 256)
        roofline = {"kernel": kname, "bound": "hbm",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": traffic_from_counters(wl.name) if default_shape else None,
                    "bytes_per_launch": wb.bwd_bytes, "avg_us": round(bwd_us, 3)}

        # Context next to the 8 TB/s peak: what the HIP runtime's own
        # device-to-device copy of one tensor (1 read + 1 write) reaches on
        # this GPU with the same rotation of buffer sets.  Not a ceiling: the
        # kernels here stream faster than it.
        if args.layout == "packed":
            def copy_one(st):
                st["dx"].copy_(st["x"])

            wb.settle(copy_one, settle_s)
            copy_us = wb.rotate_time(copy_one, R)
            runtime_copy = dict(rate(copy_us, 2 * wb.tensor_bytes),
                                kind=f"device-to-device copy of one {wb.tensor_bytes}-byte tensor "
                                     "by the HIP runtime (torch copy_; 1 read + 1 write), buffer "
                                     f"sets rotated, mean over {R} copies")
            log(f"[bench] runtime copy {copy_us:9.2f} us {runtime_copy['GB/s']:8.1f} GB/s "
                f"{100 * runtime_copy['frac']:5.1f}%")

    cpu = None
    if not args.no_cpu_baseline and args.dtype == "bf16":
        cpu = cpu_baseline(wb.inp, wl, wb.step_bytes, args.cpu_seconds)
    step_bytes = wb.step_bytes
    wb.free()
    del wb

    workloads = None
    if default_shape and wl.name == "7684x48" and not args.no_workloads:
        workloads = {}
        for name in SIDE_WORKLOADS:
            workloads[name] = side_workload(torch, binding, name, dev, settle_s)

    out = {
        "metric": "achieved HBM GB/s (% of peak) + µs, gated RMSNorm fwd/bwd at "
                  f"{wl.T}x{wl.H}x{D} {args.dtype}",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": args.dtype,
        "data": f"synthetic (seeded normal {args.dtype} inputs resident in HBM)",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "rows": rows, "D": D,
                   "layout": args.layout,
                   "eps": eps, "step": f"fwd + bwd (deterministic {args.dtype} dw)",
                   "bytes_per_step": step_bytes, "buffer_sets": nsets},
        "value_kind": "effective bandwidth: algorithmic bytes of fwd + bwd (x and g counted "
                      "in both) over the step's time; the backward may find part of x and g "
                      "that its forward just read in the 256 MB Infinity Cache. "
                      "fwd_plus_bwd_apart times the two operations apart.",
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "fwd_plus_bwd_apart": apart,
        "roofline": roofline,
        "runtime_copy": runtime_copy,
        "cpu_baseline": cpu,
        "ops": ops,
        "workloads": workloads,
        "context_r200_us": R200_7684x48_US if wl.name == "7684x48" and default_shape else None,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)


def traffic_from_counters(workload):
    """HBM bytes per launch of the backward kernel from committed counters.

    The file is written from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE)
    of this benchmark, each scaled by the same counter's reading on a copy of
    known size.  It records the workload and the SHA-256 of the kernel source
    it was taken on; for another workload, or once the source has changed,
    the figure does not apply (None).
    """
    try:
        rec = json.loads(counters_file(workload).read_text())
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload:
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_per_dispatch(path, counter):
    """{dispatch id: (kernel name, summed counter value)} from a rocprofv3 CSV."""
    import csv

    out = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            d = r["Dispatch_Id"]
            name, v = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, v + float(r["Counter_Value"]))
    return out


def summarize_counters(fetch_csv, write_csv, workload="7684x48"):
    """Per-launch HBM bytes of the kernels, scaled by a copy of known size.

    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  The benchmark's
    setup clones each input tensor with a plain device copy
    (__amd_rocclr_copyBuffer) of exactly rows * 256 bytes; the ratio of that
    size to what each counter reports for those copies is the counter's
    scale factor, applied to the other kernels' readings.
    """
    import statistics

    from silu_gated_rmsnorm_amd.inputs import WORKLOADS

    wl = WORKLOADS[workload]
    copy_bytes = wl.rows * ROW_BYTES
    fetch = _counter_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _counter_per_dispatch(write_csv, "WRITE_SIZE")

    def med(table, key):
        vals = [v for (n, v) in table.values() if key in n]
        return statistics.median(vals) if vals else None, len(vals)

    cf, ncf = med(fetch, "copyBuffer")
    cw, ncw = med(write, "copyBuffer")
    if not cf or not cw:
        sys.exit("no copy dispatches with counter values in the CSV files")
    scale_f = copy_bytes / (cf * 1024)
    scale_w = copy_bytes / (cw * 1024)
    rows = wl.rows
    alg = {"bwd_kernel": rows * 5 * ROW_BYTES + ROW_BYTES + D * 2,
           "fwd_kernel": rows * 3 * ROW_BYTES + ROW_BYTES}
    kernels = {}
    for key in ("bwd_kernel", "fwd_kernel"):
        f, nf = med(fetch, key)
        w, nw = med(write, key)
        if f is None or w is None:
            continue
        rd, wr = f * 1024 * scale_f, w * 1024 * scale_w
        kernels[key] = {"fetch_kib_raw": f, "write_kib_raw": w, "dispatches": [nf, nw],
                        "hbm_read_bytes": round(rd), "hbm_write_bytes": round(wr),
                        "hbm_bytes_per_launch": round(rd + wr),
                        "algorithmic_bytes": alg[key],
                        "traffic_over_algorithmic": round((rd + wr) / alg[key], 4)}
    rec = {"workload": workload, "kernel_source_sha256": kernel_source_sha(),
           "copy_bytes": copy_bytes, "copy_fetch_kib_raw": cf, "copy_write_kib_raw": cw,
           "copy_dispatches": [ncf, ncw],
           "fetch_scale": round(scale_f, 6), "write_scale": round(scale_w, 6),
           "kernels": kernels,
           "hbm_bytes_per_launch": kernels.get("bwd_kernel", {}).get("hbm_bytes_per_launch")}
    out = counters_file(workload)
    out.parent.mkdir(exist_ok=True)
    out.write_text(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec, indent=1))


def cpu_baseline(inp, wl, bytes_per_pass, min_seconds):
    """Time the FP64 oracle (fwd + bwd incl. dw) on the whole workload."""
    import oracle
    from silu_gated_rmsnorm_amd.inputs import bf16_bits

    b = {k: bf16_bits(v) for k, v in inp.items()}
    threads = oracle.num_threads()
    reps, total = 0, 0.0
    while total < min_seconds:
        t0 = time.perf_counter()
        oracle.fwd(b["x"], b["g"], b["w"], wl.eps)
        oracle.bwd(b["x"], b["g"], b["w"], b["dy"], wl.eps)
        total += time.perf_counter() - t0
        reps += 1
    gbps = bytes_per_pass * reps / total / 1e9
    log(f"[bench] cpu oracle: {reps} x fwd+bwd over {wl.rows} rows in {total:.1f} s, "
        f"{gbps:.2f} GB/s on {threads} threads")
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole {wl.name} workload ({wl.rows} rows), fwd + bwd with dw, "
                      f"repeated {reps} times ({total:.1f} s)",
            "seconds_per_pass": round(total / reps, 3)}


def cpu_oracle(wl, inp, passes, nbytes, repeats, chunk=1 << 20):
    """Time the FP64 oracle on a whole workload: `passes` ("fwd", "bwd") in
    order over every row, in chunks of `chunk` rows (so that its FP64
    outputs never need to be resident for the largest workloads; dw is summed
    over the chunks in order).  Host copies of the inputs are made first and
    are not timed.  Returns the median over `repeats` runs."""
    import oracle
    from silu_gated_rmsnorm_amd.inputs import bf16_bits

    b = {k: bf16_bits(v) for k, v in inp.items()}
    threads = oracle.num_threads()
    rows = wl.rows
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        for r0 in range(0, rows, chunk):
            sl = slice(r0, min(rows, r0 + chunk))
            for p in passes:
                if p == "fwd":
                    oracle.fwd(b["x"][sl], b["g"][sl], b["w"], wl.eps)
                else:
                    oracle.bwd(b["x"][sl], b["g"][sl], b["w"], b["dy"][sl], wl.eps)
        times.append(time.perf_counter() - t0)
    times.sort()
    sec = times[len(times) // 2]
    gbps = nbytes / sec / 1e9
    log(f"[bench]   oracle {'+'.join(passes)} over {rows} rows: {sec:.3f} s, {gbps:.2f} GB/s "
        f"on {threads} threads")
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole {wl.name} workload ({rows} rows), {' + '.join(passes)}, "
                      f"{'median of %d runs' % repeats if repeats > 1 else 'one run'} "
                      f"in {chunk}-row chunks",
            "seconds": round(sec, 3)}


if __name__ == "__main__":
    main()

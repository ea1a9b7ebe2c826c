"""Host logic of bench.py (CPU only): the counter scaling and when the
committed traffic figure applies.

The benchmark turns two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, KiB
per dispatch) into HBM bytes per launch by scaling each counter with its
reading on a plain copy of known size.  These tests feed hand-made CSV rows
of that format and check the arithmetic, and that the stored figure is
reported only for the workload it was taken on and only while the kernel
source is unchanged.
"""
import csv
import json

import pytest

import bench

COLUMNS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, [per-instance values])."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLUMNS)
        w.writeheader()
        for d, name, vals in rows:
            for v in vals:   # rocprofv3 may split a dispatch's counter over rows
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})
            # another counter's row on the same dispatch must be ignored
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": "OTHER",
                        "Counter_Value": 1e9})


@pytest.fixture
def counters(tmp_path, monkeypatch):
    src = tmp_path / "kernels.hip"
    src.write_text("// kernel source v1\n")
    hdr = tmp_path / "launch.h"
    hdr.write_text("// header v1\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", (src, hdr))
    monkeypatch.setattr(bench, "PROFILES_DIR", tmp_path)
    from silu_gated_rmsnorm_amd.inputs import WORKLOADS
    rows = WORKLOADS["1031x48"].rows
    copy = rows * 256                       # bytes of one BF16 [rows, 128] tensor
    # FETCH_SIZE reads half the copy's bytes, WRITE_SIZE all of them (in KiB)
    fetch_rows = [(1, "__amd_rocclr_copyBuffer", [copy / 2048 / 2] * 2),
                  (2, "__amd_rocclr_copyBuffer", [copy / 2048 / 2] * 2),
                  (3, "void grn::bwd_kernel<...>", [3 * copy / 2048]),
                  (4, "void grn::fwd_kernel<...>", [2 * copy / 2048])]
    write_rows = [(1, "__amd_rocclr_copyBuffer", [copy / 1024]),
                  (2, "__amd_rocclr_copyBuffer", [copy / 1024]),
                  (3, "void grn::bwd_kernel<...>", [2 * copy / 1024]),
                  (4, "void grn::fwd_kernel<...>", [copy / 1024])]
    _write_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch_rows)
    _write_csv(tmp_path / "w.csv", "WRITE_SIZE", write_rows)
    bench.summarize_counters(tmp_path / "f.csv", tmp_path / "w.csv", workload="1031x48")
    return {"src": src, "hdr": hdr, "copy": copy, "rows": rows,
            "rec": json.loads((tmp_path / "bwd_kernel_1031x48_traffic.json").read_text())}


def test_scaling(counters):
    rec, copy = counters["rec"], counters["copy"]
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    bwd = rec["kernels"]["bwd_kernel"]
    assert bwd["hbm_read_bytes"] == 3 * copy and bwd["hbm_write_bytes"] == 2 * copy
    fwd = rec["kernels"]["fwd_kernel"]
    assert fwd["hbm_read_bytes"] == 2 * copy and fwd["hbm_write_bytes"] == copy
    # algorithmic bytes: 5 (3) tensors plus w (and dw)
    assert bwd["algorithmic_bytes"] == 5 * copy + 256 + 256
    assert fwd["traffic_over_algorithmic"] == pytest.approx(3 * copy / (3 * copy + 256),
                                                            abs=1e-4)
    assert rec["hbm_bytes_per_launch"] == 5 * copy


def test_traffic_applies_only_to_its_workload_and_source(counters):
    assert bench.traffic_from_counters("1031x48") == 5 * counters["copy"]
    assert bench.traffic_from_counters("7684x48") is None   # no file for it here
    counters["hdr"].write_text("// header v2\n")    # any kernel source counts
    assert bench.traffic_from_counters("1031x48") is None
    counters["hdr"].write_text("// header v1\n")
    assert bench.traffic_from_counters("1031x48") == 5 * counters["copy"]
    counters["src"].write_text("// kernel source v2\n")
    assert bench.traffic_from_counters("1031x48") is None

"""CPU checks of the measurement tooling: the rocprofv3 summary tool on small
hand-written CSV files (trace medians, counter scaling by the copy control,
counter medians and ratios) and the bench's rule that counter traffic is
reported only while the kernel sources are the ones it was taken on."""

import csv
import json
import os
import types

import pytest

import bench
from bit_grouped_moe_amd import profile_summary as ps

GEMV_NAME = "void gq::grouped_gemv_kernel<false, 2, true, 0, false>(int const*)"
GEMM_NAME = "void gq::grouped_gemm_fwd_kernel<0>(gq::GemmArgs)"
COPY_NAME = "(anonymous namespace)::copy_kernel(int4 const*)"
GEMV_GRID = ps.GATE_UP_GEMV[1]
GEMM_GRID = ps.GATE_UP_GEMM[1]


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _args(**kw):
    return types.SimpleNamespace(**kw)


def test_trace_medians(tmp_path):
    fields = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Workgroup_Size_X",
              "Start_Timestamp", "End_Timestamp"]
    rows = []
    for us in (5.0, 7.0, 6.0):                              # median 6, mean 6
        rows.append({"Kernel_Name": GEMV_NAME, "Grid_Size_X": GEMV_GRID, "Grid_Size_Y": 1,
                     "Grid_Size_Z": 1, "Workgroup_Size_X": 256, "Start_Timestamp": 1000,
                     "End_Timestamp": 1000 + int(us * 1000)})
    rows.append({"Kernel_Name": "void at::native::other_kernel()", "Grid_Size_X": 64,
                 "Grid_Size_Y": 1, "Grid_Size_Z": 1, "Workgroup_Size_X": 64,
                 "Start_Timestamp": 0, "End_Timestamp": 99000})
    _write(str(tmp_path / "t" / "x_kernel_trace.csv"), fields, rows)
    out = tmp_path / "trace.md"
    ps.trace(_args(dir=str(tmp_path / "t"), cmd="cmd", title="t", out=str(out)))
    text = out.read_text()
    assert "other_kernel" not in text                      # torch's kernels are left out
    line = [l for l in text.splitlines() if "grouped_gemv_kernel" in l][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == str(GEMV_GRID) and cells[3] == "3"
    assert cells[4:8] == ["6.00", "6.00", "5.00", "7.00"]


def _counter_rows(name, grid, disp, counter, value_kib_parts):
    # rocprofv3 reports one row per counter instance; the tool sums them
    return [{"Kernel_Name": name, "Grid_Size": grid, "Dispatch_Id": disp,
             "Counter_Name": counter, "Counter_Value": v} for v in value_kib_parts]


def test_traffic_scaling_by_copy_control(tmp_path):
    fields = ["Kernel_Name", "Grid_Size", "Dispatch_Id", "Counter_Name", "Counter_Value"]
    control = 16 * 256 * 100                                 # copy_kernel grid of 100 blocks
    cgrid = 100 * 256
    # the counter reads half the bytes read and all the bytes written
    fetch = (_counter_rows(COPY_NAME, cgrid, 1, "FETCH_SIZE", [control / 2048 / 2] * 2)
             + _counter_rows(GEMV_NAME, GEMV_GRID, 2, "FETCH_SIZE", [1000.0, 1000.0])
             + _counter_rows(GEMM_NAME, GEMM_GRID, 3, "FETCH_SIZE", [5000.0]))
    write = (_counter_rows(COPY_NAME, cgrid, 1, "WRITE_SIZE", [control / 1024])
             + _counter_rows(GEMV_NAME, GEMV_GRID, 2, "WRITE_SIZE", [48.0])
             + _counter_rows(GEMM_NAME, GEMM_GRID, 3, "WRITE_SIZE", [100.0]))
    _write(str(tmp_path / "f" / "a_counter_collection.csv"), fields, fetch)
    _write(str(tmp_path / "w" / "a_counter_collection.csv"), fields, write)
    js = tmp_path / "traffic.json"
    ps.traffic(_args(fetch_dir=str(tmp_path / "f"), write_dir=str(tmp_path / "w"),
                     control_bytes=control, cmd="cmd", title="t",
                     out=str(tmp_path / "traffic.md"), json=str(js)))
    rec = json.loads(js.read_text())
    assert rec["factor_read"] == pytest.approx(2.0)
    assert rec["factor_write"] == pytest.approx(1.0)
    gv = rec["gemv_nf4_gate_up_m1"]
    assert gv["fetch_bytes"] == pytest.approx(2000.0 * 1024 * 2.0)
    assert gv["write_bytes"] == pytest.approx(48.0 * 1024)
    assert gv["source_sha256"] == ps.sources_sha("gemv_nf4_gate_up_m1")
    assert rec["gemm_nf4_gate_up_prefill"]["hbm_bytes_per_launch"] == pytest.approx(
        5000.0 * 1024 * 2.0 + 100.0 * 1024)


def test_counter_medians_and_ratios(tmp_path):
    fields = ["Kernel_Name", "Grid_Size", "Dispatch_Id", "Counter_Name", "Counter_Value"]
    rows = []
    for d, (valu, mfma, lds, conf) in enumerate([(540, 100, 160, 320), (560, 100, 170, 340),
                                                  (550, 100, 165, 330)]):
        rows += _counter_rows(GEMM_NAME, GEMM_GRID, d, "SQ_INSTS_VALU", [valu / 2, valu / 2])
        rows += _counter_rows(GEMM_NAME, GEMM_GRID, d, "SQ_INSTS_MFMA", [mfma])
        rows += _counter_rows(GEMM_NAME, GEMM_GRID, d, "SQ_INSTS_LDS", [lds])
        rows += _counter_rows(GEMM_NAME, GEMM_GRID, d, "SQ_LDS_BANK_CONFLICT", [conf])
    rows += _counter_rows(GEMV_NAME, GEMV_GRID, 9, "SQ_INSTS_VALU", [77])
    _write(str(tmp_path / "p1" / "b_counter_collection.csv"), fields, rows)
    out = tmp_path / "ctr.md"
    ps.counters(_args(dirs=[str(tmp_path / "p1")], cmd="cmd", title="t", out=str(out)))
    lines = out.read_text().splitlines()

    def row(label):
        return [c.strip() for c in [l for l in lines if l.startswith("| " + label + " ")][0]
                .strip("|").split("|")]
    assert row("SQ_INSTS_VALU")[1:] == ["77", "550"]        # medians per dispatch
    assert row("SQ_INSTS_MFMA")[1:] == ["-", "100"]
    assert row("VALU instructions per MFMA instruction")[1:] == ["-", "5.500"]
    assert row("LDS bank-conflict cycles per LDS instruction")[1:] == ["-", "2.000"]


def test_bench_reports_traffic_only_for_unchanged_sources(tmp_path, monkeypatch):
    sha = ps.sources_sha("gemv_nf4_gate_up_m1")
    rec = {"gemv_nf4_gate_up_m1": {"source_sha256": sha, "fetch_bytes": 1500.0,
                                   "write_bytes": 500.0, "hbm_bytes_per_launch": 2000.0}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    t = bench.measured_traffic("gemv_nf4_gate_up_m1", 1000.0)
    assert t == {"bytes_per_launch": 2000, "read_bytes": 1500, "written_bytes": 500,
                 "ratio_to_algorithmic": 2.0}
    assert bench.traffic_bytes(t) == 2000
    rec["gemv_nf4_gate_up_m1"]["source_sha256"] = "0" * 64   # taken on other sources
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("gemv_nf4_gate_up_m1", 1000.0) is None
    assert bench.traffic_bytes(None) is None
    assert bench.measured_traffic("gemm_nf4_gate_up_prefill", 1.0) is None   # no record

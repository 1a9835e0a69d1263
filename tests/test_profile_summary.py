"""Host logic of the measurement pipeline (CPU): the rocprofv3 summaries that
bench.py reads and the committed profiles carry, on small synthetic CSVs.

  * traffic: FETCH_SIZE / WRITE_SIZE per dispatch of the named kernel,
    scaled by what the same counter read for the 1 GiB copy;
  * stats: the timed-region average from the kernel trace and the bench
    line of the same run;
  * sweep-mfma: MfmaUtil grouped per sweep configuration;
  * bench.py reports a figure only while the sources it was taken from are
    unchanged (the SHA-256 the summary records)."""
import csv
import json
import os
import sys

import pytest

from bf16_gemm_decode_amd import profile_summary as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)
    return str(path)


def _counter_rows(counter, per_dispatch):
    """per_dispatch: [(dispatch id, kernel name, value)]"""
    return [{"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v,
             "Start_Timestamp": 1000 * d, "End_Timestamp": 1000 * d + 500} for d, k, v in per_dispatch]


def test_traffic_scales_by_the_copy_reading(tmp_path):
    fetch = _write_csv(tmp_path / "f.csv", _counter_rows("FETCH_SIZE", [
        (1, "other_kernel", 5.0), (2, "gemm_fl_kernel<0, x>", 1000.0), (3, "gemm_fl_kernel<0, x>", 3000.0)]))
    # the 1 GiB copy reads 512 KiB on this counter: the factor to bytes is 2
    fcal = _write_csv(tmp_path / "fc.csv", _counter_rows("FETCH_SIZE", [(1, "__amd_rocclr_copyBuffer", 524288.0)]))
    write = _write_csv(tmp_path / "w.csv", _counter_rows("WRITE_SIZE", [(2, "gemm_fl_kernel<0, x>", 100.0)]))
    wcal = _write_csv(tmp_path / "wc.csv", _counter_rows("WRITE_SIZE", [(1, "copyBuffer", 1048576.0)]))
    out = tmp_path / "t.json"
    ps.main(["traffic", "--fetch", fetch, "--fetch-cal", fcal, "--write", write, "--write-cal", wcal,
             "--kernel", "gemm_fl_kernel<0", "--source", "gemm.hip", "common.hpp", "--out", str(out),
             "--commands", "c"])
    t = json.load(open(out))
    assert t["fetch_size"]["dispatches"] == 2
    assert t["fetch_size"]["bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2.0)
    assert t["write_size"]["bytes_per_launch"] == pytest.approx(100.0 * 1024)
    assert t["beyond_l2_bytes_per_launch"] == pytest.approx(2000.0 * 2048 + 100.0 * 1024)
    assert t["kernel_sources_sha256"] == ps.source_digest(["gemm.hip", "common.hpp"])


def test_counters_per_kernel_label(tmp_path):
    a = _write_csv(tmp_path / "a.csv", _counter_rows("TA_BUSY_avr", [
        (1, "batch_rows_kernel<1, 1>", 10.0), (2, "attn_segment_kernel<256, 4>", 4.0),
        (3, "batch_rows_kernel<1, 1>", 30.0)]))
    b = _write_csv(tmp_path / "b.csv", _counter_rows("MemUnitStalled", [(1, "batch_rows_kernel<1, 1>", 2.0)]))
    out = tmp_path / "c.json"
    ps.main(["counters", "--csv", a, b, "--kernel", "rows=batch_rows_kernel", "attn=attn_segment",
             "--source", "batch.hip", "--out", str(out), "--commands", "c"])
    c = json.load(open(out))
    rows = c["kernels"]["rows"]["counters"]
    assert rows["TA_BUSY_avr"] == {"mean": 20.0, "min": 10.0, "max": 30.0, "dispatches": 2}
    assert rows["MemUnitStalled"]["mean"] == 2.0
    assert c["kernels"]["attn"]["counters"]["TA_BUSY_avr"]["dispatches"] == 1
    assert c["kernels"]["rows"]["avg_duration_ns"] == 500
    with pytest.raises(SystemExit):
        ps.main(["counters", "--csv", a, "--kernel", "x=no_such_kernel", "--source", "batch.hip",
                 "--out", str(out), "--commands", "c"])


def test_timed_region_and_bench_line(tmp_path):
    stats = _write_csv(tmp_path / "s.csv", [{"Name": "gemm_fl_kernel<0, y>", "Calls": 5, "AverageNs": 1.0}])
    # dispatches of the GEMM: two warm-ups of 3000 ns, then 1000, 1100, 1200
    trace = _write_csv(tmp_path / "k.csv", [
        {"Dispatch_Id": d, "Kernel_Name": k, "Start_Timestamp": 10000 * d, "End_Timestamp": 10000 * d + t}
        for d, k, t in [(1, "gemm_fl_kernel<0, y>", 3000), (2, "gemv_kernel", 50), (3, "gemm_fl_kernel<0, y>", 3000),
                        (4, "gemm_fl_kernel<0, y>", 1000), (5, "gemm_fl_kernel<0, y>", 1100),
                        (6, "gemm_fl_kernel<0, y>", 1200)]])
    bench = tmp_path / "b.out"
    bench.write_text("noise\n" + json.dumps({"roofline": {"avg_launch_ms": 0.0011}, "gemv": {"avg_launch_us": 0.05}}) + "\n")
    out = tmp_path / "s.txt"
    ps.main(["stats", stats, str(out), "--command", "c", "--trace", trace, "--timed", "gemm_fl_kernel<0:2:3",
             "--bench-json", str(bench)])
    text = open(out).read()
    assert "dispatches 2..4 of 5: average 1100.0 ns, min 1000, max 1200" in text
    assert "avg_launch_ms 0.0011" in text


def test_sweep_mfma_groups_dispatches_by_configuration(tmp_path):
    cfgs = [{"shape": [64, 64, 64], "dtype": "bf16", "a_layout": "m-major", "tile": t, "tile_mnk": [256, 256, 32],
             "group_m": 8, "ms": 1.0, "tflops": 1.0} for t in (16, 10)]
    sweep = tmp_path / "sw.json"
    sweep.write_text("\n".join(json.dumps(c) for c in cfgs) + "\n")
    # per configuration: 1 + warmup 1 + reps 2 dispatches; the data-generation
    # kernels in between are not GEMMs
    rows, d = [], 0
    for base in (50.0, 20.0):
        d += 1
        rows.append((d, "fill_kernel", 99.0))
        for j, v in enumerate((0.0, 0.0, base, base + 10.0)):
            d += 1
            rows.append((d, "gemm_fl_kernel<1, z>", v))
    util = _write_csv(tmp_path / "u.csv", _counter_rows("MfmaUtil", rows))
    out = tmp_path / "m.md"
    ps.main(["sweep-mfma", "--util-csv", util, "--sweep-json", str(sweep), "--warmup", "1", "--reps", "2",
             "--out", str(out), "--command", "c"])
    lines = [l for l in open(out) if l.startswith("| 64x64x64")]
    assert lines[0].rstrip().endswith("| 55.0 |") and lines[1].rstrip().endswith("| 25.0 |")


def test_bench_reports_counters_only_for_unchanged_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    srcs = ["gemm.hip", "common.hpp"]
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = {"kernel_sources": srcs, "kernel_sources_sha256": ps.source_digest(srcs), "beyond_l2_bytes_per_launch": 7.0,
            "kernels": {"k": {"mfma_util_percent": {"mean": 12.345}}}}
    stale = dict(good, kernel_sources_sha256="0" * 64)
    (prof / "good.json").write_text(json.dumps(good))
    (prof / "stale.json").write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(srcs, "good.json") == 7.0
    assert bench.measured_traffic(srcs, "stale.json") is None
    assert bench.measured_traffic(srcs + ["api.hip"], "good.json") is None     # other source list
    assert bench.measured_traffic(srcs, "missing.json") is None
    assert bench.measured_mfma_util(srcs, "good.json", "k") == 12.35
    assert bench.measured_mfma_util(srcs, "stale.json", "k") is None

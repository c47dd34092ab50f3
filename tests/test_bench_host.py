"""Host logic of bench.py, on the CPU: the rocprofv3 summaries it builds
(marker window, per-kernel means, calibration ratio), the guard that drops
counter-measured traffic once a kernel's sources change, the one-GPU
refusal, and the algorithmic byte counts the roofline divides by."""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _trace_rows():
    """Dispatches 1..7: kernels outside the markers, two markers, the
    kernels between them and the calibration copy last in the window."""
    def r(i, name, grid, t0, t1):
        return {"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid,
                "Start_Timestamp": t0, "End_Timestamp": t1}
    return [
        r(1, "void kvq::(anonymous namespace)::encode128_kernel<0, 0, 0>(kvq::CodecArgs)", 458752, 0, 99000),
        r(2, "void at::native::sleep(long)", 1, 100000, 101000),
        r(3, "void kvq::(anonymous namespace)::encode128_kernel<0, 0, 0>(kvq::CodecArgs)", 458752, 102000, 137000),
        r(4, "void kvq::(anonymous namespace)::encode128_kernel<0, 0, 0>(kvq::CodecArgs)", 458752, 140000, 177000),
        r(5, "void kvq::(anonymous namespace)::decode128_kernel<0, 0>(kvq::CodecArgs)", 458752, 180000, 210000),
        r(6, "__amd_rocclr_copyBuffer", 131072, 220000, 440000),
        r(7, "void at::native::sleep(long)", 1, 450000, 451000),
    ]


def test_trace_summary_window_and_means(tmp_path):
    p = tmp_path / "kernel_trace.csv"
    _write_csv(p, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"], _trace_rows())
    out = bench.trace_summary(str(p))
    rows = {l.split("|")[1].strip(): [x.strip() for x in l.split("|")[2:-1]]
            for l in out.splitlines()[2:]}
    # the 99 us dispatch before the first marker is outside the window
    assert rows["encode128_kernel<0, 0, 0>"] == ["458752", "2", "36.00", "35.00", "37.00"]
    assert rows["decode128_kernel<0, 0>"] == ["458752", "1", "30.00", "30.00", "30.00"]
    assert rows["calibration copy (512 MiB)"][1:3] == ["1", "220.00"]
    assert not any("sleep" in k for k in rows)


def test_trace_summary_counters_and_calibration(tmp_path):
    p = tmp_path / "counter_collection.csv"
    base = _trace_rows()
    rows = []
    for r in base:
        for ctr, val in (("FETCH_SIZE", 1000.0), ("WRITE_SIZE", 500.0)):
            v = val
            if r["Dispatch_Id"] == 6:      # the calibration copy: 512 MiB read, 512 MiB written
                v = 262144.0 if ctr == "FETCH_SIZE" else 524288.0
            if r["Dispatch_Id"] == 4:
                v *= 3
            # two rows per dispatch and counter (per-XCD partial sums) add up
            for half in (v / 2, v / 2):
                rows.append({"Dispatch_Id": r["Dispatch_Id"], "Kernel_Name": r["Kernel_Name"],
                             "Grid_Size": r["Grid_Size"], "Counter_Name": ctr, "Counter_Value": half})
    _write_csv(p, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"], rows)
    out = bench.trace_summary(str(p))
    got = {}
    for l in out.splitlines()[2:]:
        c = [x.strip() for x in l.split("|")[1:-1]]
        got[(c[0], c[2])] = c
    assert got[("encode128_kernel<0, 0, 0>", "FETCH_SIZE")][3:5] == ["2", "2000.0"]
    assert got[("encode128_kernel<0, 0, 0>", "WRITE_SIZE")][4] == "1000.0"
    assert got[("calibration copy (512 MiB)", "FETCH_SIZE")][5] == "0.5000"
    assert got[("calibration copy (512 MiB)", "WRITE_SIZE")][5] == "1.0000"


def test_trace_summary_needs_two_markers(tmp_path):
    p = tmp_path / "kernel_trace.csv"
    _write_csv(p, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"],
               _trace_rows()[:3])
    with pytest.raises(SystemExit):
        bench.trace_summary(str(p))


def test_measured_traffic_follows_the_sources(monkeypatch):
    import hashlib
    h = hashlib.sha256()
    for f in bench.TRAFFIC["attn"]["files"]:
        with open(os.path.join(ROOT, "kv_cache_int4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    # counters recorded on the sources as they stand are reported ...
    monkeypatch.setitem(bench.TRAFFIC, "attn", dict(bench.TRAFFIC["attn"], sha256=h.hexdigest()[:16]))
    assert bench.measured_traffic("attn") == round(bench.TRAFFIC["attn"]["bytes"])
    # ... and dropped once the sources differ from those the counters were taken on
    monkeypatch.setitem(bench.TRAFFIC, "attn", dict(bench.TRAFFIC["attn"], sha256="0000000000000000"))
    assert bench.measured_traffic("attn") is None


def test_recorded_traffic_is_near_the_algorithmic_bytes():
    # the recorded counters are within 2% of the algorithmic bytes: nothing
    # is re-read
    attn = 64 * 2 * 32769 * 2 * (64 + 8)
    codec = 458752 * (256 + 64 + 8)
    assert attn == 603998208
    assert abs(bench.TRAFFIC["attn"]["bytes"] / attn - 1) < 0.02
    assert abs(bench.TRAFFIC["encode"]["bytes"] / codec - 1) < 0.02
    assert abs(bench.TRAFFIC["decode"]["bytes"] / codec - 1) < 0.02


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr

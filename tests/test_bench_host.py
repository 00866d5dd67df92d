"""Host-side logic of the benchmark, no GPU: the single-GPU guard, and the
arithmetic that turns rocprofv3 output into the committed summaries (counter
calibration, XCD normalisation, the source-hash guard on the traffic
figure), checked on small hand-made CSV files."""
import argparse
import csv
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
VOCAB = "void gq::qmv_kernel<8, 0, 2, 1, 4, false>(gq::QmvParams)"
COPY = "__amd_rocclr_copyBuffer"
FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kern, grid, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Grid_Size": grid, "Kernel_Name": kern, "Counter_Name": counter,
                        "Counter_Value": value})


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_pmc_summary_calibrates_against_the_copy(tmp_path, capsys):
    # the copy's counter reads half its true size (factor 2) for FETCH_SIZE,
    # the true size for WRITE_SIZE; the largest copy dispatch is the reference
    kib = bench.COPY_BYTES / 1024.0
    fetch = [(COPY, 1024, "FETCH_SIZE", 3.0), (COPY, 1 << 24, "FETCH_SIZE", kib / 2),
             (COPY, 1 << 24, "FETCH_SIZE", kib / 2)]
    fetch += [(VOCAB, 262144, "FETCH_SIZE", v) for v in (1000.0, 1002.0, 998.0)]
    write = [(COPY, 1 << 24, "WRITE_SIZE", kib)] + [(VOCAB, 262144, "WRITE_SIZE", 512.0)] * 3
    _write_counters(str(tmp_path / "f"), fetch)
    _write_counters(str(tmp_path / "w"), write)
    bench.pmc_summary(argparse.Namespace(pmc_summary="%s,%s" % (tmp_path / "f", tmp_path / "w"),
                                         write_profile=False))
    out = dict(line.split(" = ", 1) for line in capsys.readouterr().out.splitlines() if " = " in line)
    assert float(out["fetch_calibration_factor"]) == pytest.approx(2.0)
    assert float(out["write_calibration_factor"]) == pytest.approx(1.0)
    assert float(out["fetch_bytes_per_launch"]) == pytest.approx(1000.0 * 1024 * 2, abs=1)
    assert float(out["write_bytes_per_launch"]) == pytest.approx(512.0 * 1024, abs=1)
    alg = 262144 * 64 * 34 + 2048 * 4 + 262144 * 4
    assert int(out["algorithmic_bytes_per_launch"]) == alg
    assert out["kernel_source_hash"] == bench.kernel_source_hash()


def test_traffic_is_null_unless_taken_from_these_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic() is None                      # missing
    body = "# header = ignored\nfetch_bytes_per_launch = 100\nwrite_bytes_per_launch = 20\n"
    f.write_text(body + "kernel_source_hash = %s\n" % bench.kernel_source_hash())
    assert bench.load_traffic() == 120.0
    f.write_text(body + "kernel_source_hash = 0123456789abcdef\n")
    assert bench.load_traffic() is None                      # other kernel sources


def test_counter_summary_normalises_grbm_over_xcds(tmp_path, capsys):
    # one kernel: 8 XCDs x 1000 active cycles; VALU busy 500 quad-cycles per CU
    # -> 50 %; MFMA busy 250 cycles per SIMD -> 25 %
    grbm = 8 * 1000.0
    a = [(VOCAB, 262144, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 250.0), (VOCAB, 262144, "SQ_INSTS_VALU_MFMA_MOPS_I8", 7.0),
         (VOCAB, 262144, "GRBM_GUI_ACTIVE", grbm)]
    b = [(VOCAB, 262144, "SQ_ACTIVE_INST_VALU", 256 * 500.0), (VOCAB, 262144, "SQ_INSTS_VALU", 42.0),
         (VOCAB, 262144, "GRBM_GUI_ACTIVE", grbm)]
    _write_counters(str(tmp_path / "a"), a)
    _write_counters(str(tmp_path / "b"), b)
    bench.counters_summary(argparse.Namespace(counters_summary="%s,%s" % (tmp_path / "a", tmp_path / "b"),
                                              write_profile=False))
    line = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("qmv Q8_0 fp32 x, tall: vocab")][0]
    fields = line.split()
    assert "50.0%" in fields and "25.00%" in fields


def test_stats_summary_reports_the_dominant_kernel(tmp_path, capsys):
    d = tmp_path / "prof"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([VOCAB, 10, 860000, 86000.0, 90.0, 85000, 87000, 1.0])
        w.writerow([COPY, 2, 8000, 4000.0, 1.0, 3000, 5000, 1.0])
    (tmp_path / "prof.log").write_text('{"roofline": {"avg_launch_us": 87.72}}\n')
    bench.stats_summary(argparse.Namespace(stats_summary=str(d), write_profile=False))
    out = capsys.readouterr().out
    alg = 262144 * 64 * 34 + 2048 * 4 + 262144 * 4
    assert "%d B / 86.00 us = %.2f TB/s" % (alg, alg / 86.0 / 1e6) in out
    assert "87.72 us" in out and "difference 2.0%" in out
    assert out.index("vocab") < out.index("runtime copy")    # sorted by total time


def test_stats_summary_averages_the_timed_region_from_the_trace(tmp_path, capsys):
    # 2 warm-up and 3 timed vocab launches, then a later (untimed) one; the
    # profiled run's events read 90 us, the unprofiled run's 88 us
    d = tmp_path / "prof"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([VOCAB, 6, 600000, 100000.0, 90.0, 80000, 200000, 1.0])
    durs = [200000, 100000, 86000, 86000, 86000, 42000]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerow([1, COPY, 0, 5000])
        # written out of dispatch order: the summary sorts by Dispatch_Id
        for i, dur in reversed(list(enumerate(durs))):
            w.writerow([10 + i, VOCAB, 1000000 * i, 1000000 * i + dur])
    (tmp_path / "prof.log").write_text('[bench] x\n{"warmup": 2, "steps": 3, "roofline": {"avg_launch_us": 90.3}}\n')
    plain = tmp_path / "plain.json"
    plain.write_text('{"warmup": 2, "steps": 3, "roofline": {"avg_launch_us": 87.72, "frac": 0.81}}\n')
    bench.stats_summary(argparse.Namespace(stats_summary="%s,%s" % (d, plain), write_profile=False))
    out = capsys.readouterr().out
    assert "timed region's launches" in out and "B / 86.00 us" in out
    assert "90.30 us" in out and "difference 5.0%" in out
    assert "87.72 us" in out and "difference 2.0%" in out and "0.810" in out


def test_stats_summary_compares_events_with_the_bracketed_launches(tmp_path, capsys):
    # 1 warm-up and 4 timed vocab launches; the events bracket every 2nd timed
    # one (launches 1 and 3 of the region: 86 us each, the others 96 us)
    d = tmp_path / "prof"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([VOCAB, 5, 500000, 100000.0, 90.0, 86000, 136000, 1.0])
    durs = [136000, 86000, 96000, 86000, 96000]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, dur in enumerate(durs):
            w.writerow([10 + i, VOCAB, 1000000 * i, 1000000 * i + dur])
    (tmp_path / "prof.log").write_text('{"warmup": 1, "steps": 4, "roofline": {"avg_launch_us": 87.72, '
                                       '"event_every": 2}}\n')
    bench.stats_summary(argparse.Namespace(stats_summary=str(d), write_profile=False))
    out = capsys.readouterr().out
    assert "B / 91.00 us" in out                       # every timed launch
    assert "one in 2 of them" in out and "86.00 us" in out
    assert "87.72 us" in out and "difference 2.0%" in out


def test_step_traffic_summary_matches_launches_and_calibrates(tmp_path, capsys):
    # a step of two launches, run twice, then the calibration copy; the copy
    # reads 2x its bytes on FETCH_SIZE (factor 0.5) and 1x on WRITE_SIZE
    tile = "void gq::(anonymous namespace)::tile_kernel<1, true>(unsigned char const*)"
    kib = bench.COPY_BYTES / 1024.0
    launches = [["qmv_q8_0 vocab", 1000, 24], ["tile M=8", 2000, 48]]
    fetch = [(COPY, 512, 1.0)] + [(VOCAB, 262144, 2.0), (tile, 262144, 4.0)] * 2 + [(COPY, 1 << 20, 2 * kib)] * 3
    write = [(COPY, 512, 1.0)] + [(VOCAB, 262144, 0.5), (tile, 262144, 1.0)] * 2 + [(COPY, 1 << 20, kib)] * 3
    _write_counters(str(tmp_path / "f"), [(k, g, "FETCH_SIZE", v) for k, g, v in fetch])
    _write_counters(str(tmp_path / "w"), [(k, g, "WRITE_SIZE", v) for k, g, v in write])
    (tmp_path / "f.log").write_text('[bench] x\n{"step_launches": %s, "steps": 2}\n' % str(launches).replace("'", '"'))
    bench.step_traffic_summary(argparse.Namespace(step_traffic_summary="%s,%s" % (tmp_path / "f", tmp_path / "w"),
                                                  write_profile=False))
    out = capsys.readouterr().out.splitlines()
    vocab = [ln for ln in out if ln.startswith("qmv_q8_0 vocab")][0].split()
    tile_ln = [ln for ln in out if ln.startswith("tile M=8")][0].split()
    # fetch 2 KiB x 0.5 = 1024 B, write 0.5 KiB x 1 = 512 B, against 1024 algorithmic bytes
    assert vocab[-4:] == ["1024", "512", "1024", "1.500"]
    assert tile_ln[-4:] == ["2048", "1024", "2048", "1.500"]

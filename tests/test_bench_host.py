"""Host logic of bench.py (no GPU): the multi-GPU refusal, and the summary of
a profiling session's raw rocprofv3 output into the traffic figure, with the
counters scaled by what they read for a copy of known size."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counter_rows(kernel, counter, per_dispatch):
    """Two partial readings per dispatch (as rocprofv3 lists them per block),
    summing to the given totals."""
    rows = []
    for i, total in enumerate(per_dispatch):
        rows.append([i + 1, kernel, counter, total * 0.25])
        rows.append([i + 1, kernel, counter, total * 0.75])
    return rows


@pytest.fixture
def session(tmp_path, monkeypatch):
    out = tmp_path / "raw"
    kern = "void fa::(anonymous namespace)::fwd_bf16_kernel<128, 1, true, false>(...)"
    _csv(str(out / "trace" / "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
         [[kern, 600, 1950000.0, 1900000.0, 2500000.0], ["void copy_kernel(...)", 5, 1000.0, 900.0, 1100.0]])
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _csv(str(out / "fetch" / "run_counter_collection.csv"), hdr, _counter_rows(kern, "FETCH_SIZE", [800000.0, 820000.0]))
    _csv(str(out / "write" / "run_counter_collection.csv"), hdr, _counter_rows(kern, "WRITE_SIZE", [130000.0, 130000.0]))
    # a 256 MiB copy: FETCH_SIZE reads half the copied KiB, WRITE_SIZE all of them
    _csv(str(out / "copy_fetch" / "run_counter_collection.csv"), hdr,
         _counter_rows("void at::native::copy_kernel(...)", "FETCH_SIZE", [131072.0] * 5))
    _csv(str(out / "copy_write" / "run_counter_collection.csv"), hdr,
         _counter_rows("void at::native::copy_kernel(...)", "WRITE_SIZE", [262144.0] * 5))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "profiles" / "traffic.json"))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda names=None: "0123456789abcdef")
    return tmp_path, str(out)


def test_summary_scales_counters_by_the_copy(session, capsys):
    tmp, out = session
    bench.summarize(out, "wl")
    t = json.load(open(str(tmp / "profiles" / "traffic.json")))["wl"]
    cal = t["copy_calibration"]
    assert cal["fetch_factor"] == pytest.approx(2.0) and cal["write_factor"] == pytest.approx(1.0)
    assert t["fetch_kib_per_launch"] == pytest.approx(810000.0)
    assert t["read_bytes_per_launch"] == pytest.approx(810000.0 * 1024 * 2.0)
    assert t["write_bytes_per_launch"] == pytest.approx(130000.0 * 1024)
    assert t["bytes_per_launch"] == pytest.approx(t["read_bytes_per_launch"] + t["write_bytes_per_launch"])
    trace = open(str(tmp / "profiles" / "fa_fwd_bf16_wl_kernel_trace.txt")).read()
    assert "average=1950.0 us" in trace and "0123456789abcdef" in trace
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert line["kernel_avg_us"] == pytest.approx(1950.0)


def test_traffic_reported_only_for_the_same_source_and_workload(session, monkeypatch):
    tmp, out = session
    bench.summarize(out, "wl")
    assert bench.measured_traffic("wl") == pytest.approx((810000.0 * 2.0 + 130000.0) * 1024)
    assert bench.measured_traffic("other") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda names=None: "fedcba9876543210")
    assert bench.measured_traffic("wl") is None


def test_summary_keeps_other_workloads(session):
    tmp, out = session
    bench.summarize(out, "wl")
    bench.summarize(out, "wl2")
    t = json.load(open(str(tmp / "profiles" / "traffic.json")))
    assert set(t) == {"wl", "wl2"}
    assert bench.measured_traffic("wl2") == pytest.approx(bench.measured_traffic("wl"))


def test_per_kernel_counters_average_a_counter_of_both_passes(session):
    """GRBM_GUI_ACTIVE is collected in both counter passes of a path; with the
    dispatch ids of the two runs alike, it is averaged, not summed."""
    tmp, out = session
    kern = "void fa::(anonymous namespace)::fwd_fp8_kernel<128, true>(...)"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _csv(os.path.join(out, "fp8_sq", "run_counter_collection.csv"), hdr,
         _counter_rows(kern, "GRBM_GUI_ACTIVE", [8e6, 8e6]) + _counter_rows(kern, "SQ_VALU_MFMA_BUSY_CYCLES", [512e6, 512e6]))
    _csv(os.path.join(out, "fp8_sq2", "run_counter_collection.csv"), hdr,
         _counter_rows(kern, "GRBM_GUI_ACTIVE", [8e6, 8e6]) + _counter_rows(kern, "SQ_INSTS_MFMA", [1e6, 1e6]))
    bench.summarize(out, "wl")
    txt = open(str(tmp / "profiles" / "fa_fwd_fp8_bf16_n16k_d128_causal_amplified_counters.txt")).read()
    assert "GRBM_GUI_ACTIVE              8e+06" in txt
    # 512e6 busy cycles over (8e6 / 8 XCDs) cycles x 1024 SIMDs
    assert "MFMA busy = 50.0 %" in txt


def test_io_models_match_the_pages_formulas():
    """Per head: 4N^2 + 4Nd elements for the three-pass attention and
    8 N^2 d^2 / M for the tiled pass (M elements of on-chip memory)."""
    from io_aware_softmax_fwd_amd import workloads as W
    w = W.WORKLOADS[4]
    m = bench.io_models(w)
    N, d, heads = 16384, 128, 32
    assert m["algorithmic"] == heads * (4 * N * d * 2 + 4 * N)
    assert m["standard_4N2_4Nd"] == heads * (4 * N * N + 4 * N * d) * 2
    assert m["tiled_8N2d2_over_M"] == pytest.approx(heads * 8 * N * N * d * d / (160 * 1024 / 2) * 2)
    # causal: query tile t reads keys [0, 128 (t+1)) of K and of V
    kv = sum(128 * (t + 1) for t in range(N // 128))
    assert m["kv_per_query_tile"] == heads * (2 * kv * d * 2 + 2 * N * d * 2 + 4 * N)
    w2 = W.WORKLOADS[5]
    m2 = bench.io_models(w2)
    tiles = -(-32749 // 128)
    assert m2["kv_per_query_tile"] == 16 * (2 * tiles * 32749 * 64 * 2 + 2 * 32749 * 64 * 2 + 4 * 32749)


def test_untimed_steps_run_warmup_then_settle():
    calls = []
    n = bench.run_untimed(lambda: calls.append(1), lambda: None, 3, 0.0)
    assert n == 0 and len(calls) == 3
    calls.clear()
    n = bench.run_untimed(lambda: calls.append(1), lambda: None, 2, 20.0)
    assert n > 0 and n % 8 == 0 and len(calls) == 2 + n

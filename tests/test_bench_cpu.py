"""bench.py's host logic without a GPU: the work a launch label stands for,
and the parsing of rocprofv3 CSV output (kernel trace and counter runs)
into per-label durations, traffic and roofline objects.  The CSV files are
written here in rocprofv3's column layout."""
import csv
import json
import os

import pytest

import bench


def test_label_work_decode_and_prefill():
    assert bench.label_work("gemv", "gate_up") == (bench.packed_bytes(37888, 3584), "GB/s",
                                                   bench.HBM_PEAK_GBPS)
    assert bench.label_work("gemv", "dom:int4:gate_up")[0] == bench.awq_packed_bytes(37888, 3584)
    assert bench.label_work("gemv", "m2:lm_head")[0] == bench.packed_bytes(152064, 3584)
    assert bench.label_work("gemv", "vx:w13")[0] == bench.packed_bytes(18432, 3072)
    assert bench.label_work("gemv", "u:k")[0] == bench.packed_bytes(512, 3584)
    assert bench.label_work("gemm", "qkv")[0] == 2 * 1024 * 4608 * 3584
    assert bench.label_work("gemm", "t113:down")[0] == 2 * 113 * 3584 * 18944
    assert bench.label_work("gemm", "c29:o")[0] == 2 * 29 * 3584 * 3584
    assert bench.label_work("gemm", "pmc:c29:down")[0] == 2 * 29 * 3584 * 18944
    assert bench.label_work("gemm", "c4:gate_up")[0] == 2 * 1024 * 37888 * 3584
    assert bench.label_work("gemm", "c4t:qkv")[0] == 2 * 113 * 4608 * 3584
    assert bench.label_work("gemv", "nonsense") is None


def _write(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


GEMV = "void nf4::(anonymous namespace)::gemv_fast_kernel<1, false, false>(unsigned short const*)"
GEMM = "void nf4::(anonymous namespace)::gemm_wide_kernel<4, false>(unsigned short const*)"
ZERO = "nf4::(anonymous namespace)::zero_counters_kernel(unsigned int*, long)"


@pytest.fixture
def prof(tmp_path):
    """A fake profiler result: trace (2 gemv + 1 gemm labelled, other kernels
    interleaved) and fetch/write counter runs with the copy calibration."""
    base = tmp_path
    (base / "trace").mkdir()
    _write(base / "trace" / "run_kernel_trace.csv",
           ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [{"Kernel_Name": GEMV, "Start_Timestamp": 100, "End_Timestamp": 18100},
            {"Kernel_Name": "at::native::fill", "Start_Timestamp": 20000, "End_Timestamp": 21000},
            {"Kernel_Name": GEMV, "Start_Timestamp": 30000, "End_Timestamp": 50000},
            {"Kernel_Name": ZERO, "Start_Timestamp": 60000, "End_Timestamp": 64000},
            {"Kernel_Name": GEMM, "Start_Timestamp": 70000, "End_Timestamp": 370000}])
    json.dump([["gemv", "dom:gate_up"], ["gemv", "dom:gate_up"], ["gemm", "dom:gate_up"]],
              open(base / "trace_launches.json", "w"))
    for key, counter, copy, g, m in (("fetch", "FETCH_SIZE", 524288, 40000, 160000),
                                     ("write", "WRITE_SIZE", 1048576, 100, 150000)):
        (base / key).mkdir()
        _write(base / key / "run_counter_collection.csv",
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
               [{"Dispatch_Id": 1, "Kernel_Name": bench.COPY_KERNEL, "Counter_Name": counter,
                 "Counter_Value": copy},
                {"Dispatch_Id": 3, "Kernel_Name": GEMM, "Counter_Name": counter,
                 "Counter_Value": m},
                {"Dispatch_Id": 2, "Kernel_Name": GEMV, "Counter_Name": counter,
                 "Counter_Value": g}])
        json.dump([["gemv", "pmc:gate_up"], ["gemm", "pmc:gate_up"]],
                  open(base / (key + "_launches.json"), "w"))
    p = {"dir": str(base), "commands": {"trace": "t", "fetch": "f", "write": "w"}}
    p["trace"] = bench.labelled_durations(str(base / "trace"), str(base / "trace_launches.json"))
    p["fetch"] = bench.labelled_counters(str(base / "fetch"), str(base / "fetch_launches.json"),
                                         "FETCH_SIZE")
    p["write"] = bench.labelled_counters(str(base / "write"), str(base / "write_launches.json"),
                                         "WRITE_SIZE")
    return p


def test_durations_and_traffic(prof):
    names, v = prof["trace"][("gemv", "dom:gate_up")]
    assert v == [18000, 20000] and names == {"gemv_fast_kernel<1, false, false>"}
    assert prof["trace"][("gemm", "dom:gate_up")][1] == [300000]
    assert bench.rocprof_mean_us(prof, ("gemv", "dom:gate_up"))[0] == pytest.approx(19.0)
    # FETCH_SIZE reads half the copy's bytes: scale x2; WRITE_SIZE x1
    assert bench.traffic_bytes(prof, ("gemv", "pmc:gate_up")) == 40000 * 2048 + 100 * 1024
    assert bench.traffic_bytes(prof, ("gemv", "missing")) is None


def test_roofline_entry_uses_the_rocprof_mean(prof):
    r = bench.roofline_entry(prof, "dom:gate_up", 17.0, 76382208, 8000.0, "GB/s", "hbm", "k",
                             "algorithmic_bytes")
    assert r["rocprof_mean_us"] == pytest.approx(19.0)
    assert r["achieved"] == pytest.approx(76382208 / 19e-6 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)
    assert r["event_us"] == 17.0 and r["traffic"] == 40000 * 2048 + 100 * 1024
    g = bench.roofline_entry(prof, "dom:gate_up", 290.0, 278099132416, 2500.0, "TFLOP/s", "mfma",
                             "k", "algorithmic_flop")
    assert g["achieved"] == pytest.approx(278099132416 / 300e-6 / 1e12, rel=1e-4)
    e = bench.roofline_entry({"error": "x"}, "dom:gate_up", 20.0, 80e6, 8000.0, "GB/s", "hbm",
                             "k", "algorithmic_bytes")
    assert e["rocprof_mean_us"] is None and e["achieved"] == pytest.approx(4000.0)
    assert e["traffic"] is None and "events only" in e["timed_on"]


def test_launch_log_mismatch_is_an_error(tmp_path, prof):
    bad = tmp_path / "bad.json"
    json.dump([["gemv", "a"]], open(bad, "w"))
    with pytest.raises(RuntimeError):
        bench.labelled_durations(os.path.join(prof["dir"], "trace"), str(bad))


def test_write_profiles(tmp_path, prof):
    out = tmp_path / "out"
    bench.write_profiles(prof, str(out))
    text = (out / "dominant_kernels_gate_up.md").read_text()
    assert "dom:gate_up" in text and "HBM traffic per launch" in text
    assert prof["dir"] not in text.split("\n", 1)[1]  # temporary paths read <tmp>


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus above 1 (or a WORLD_SIZE above 1)
    exits with status 2 and a message, before touching a GPU or rocprofv3."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv],
                           capture_output=True, text=True, timeout=120,
                           env={**os.environ, **env})
        assert r.returncode == 2, (argv, env, r.returncode, r.stderr[-500:])
        assert "one GPU" in r.stderr
        assert r.stdout == ""

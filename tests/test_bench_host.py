"""Host-side logic of bench.py: the counter summary (copy calibration, per-dispatch
scaling) and the source-hash guard that keeps stale traffic figures out of the
bench line.  Runs on CPU with synthetic CSV files shaped like rocprofv3's."""
import csv
import importlib.util
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench(tmp_path, monkeypatch):
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    monkeypatch.setitem(sys.modules, "bench_mod", mod)   # (the CPU baseline's workers look it up)
    spec.loader.exec_module(mod)
    monkeypatch.setattr(mod, "PROFILES", str(tmp_path / "profiles"))
    monkeypatch.setattr(mod, "TRAFFIC_FILE", str(tmp_path / "profiles" / "traffic.txt"))
    return mod


def write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def fake_profiles(tmp_path, fetch_copy=524288.0, write_copy=1048576.0):
    kt = tmp_path / "kt"
    write_csv(str(kt / "x_kernel_stats.csv"), ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage",
                                               "MinNs", "MaxNs", "StdDev"],
              [{"Name": "void gdn::chunk_kernel<128, 128, false, unsigned short, 2>(gdn::SeqLaunch)", "Calls": 7,
                "TotalDurationNs": 7e6, "AverageNs": 1e6, "Percentage": 50, "MinNs": 9e5, "MaxNs": 1.1e6,
                "StdDev": 1}])
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    fetch_rows = [
        {"Kernel_Name": "vectorized_elementwise_kernel<MulFunctor<float>>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 12.0},
        {"Kernel_Name": "vectorized_elementwise_kernel<MulFunctor<float>>", "Counter_Name": "FETCH_SIZE", "Counter_Value": fetch_copy},
        {"Kernel_Name": "chunk_kernel<128, 128, false, unsigned short, 2>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
        {"Kernel_Name": "chunk_kernel<128, 128, false, unsigned short, 2>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0},
        {"Kernel_Name": "recurrent_kernel<128, 128, unsigned short, unsigned short>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 50.0},
    ]
    write_rows = [
        {"Kernel_Name": "vectorized_elementwise_kernel<MulFunctor<float>>", "Counter_Name": "WRITE_SIZE", "Counter_Value": write_copy},
        {"Kernel_Name": "chunk_kernel<128, 128, false, unsigned short, 2>", "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0},
        {"Kernel_Name": "recurrent_kernel<128, 128, unsigned short, unsigned short>", "Counter_Name": "WRITE_SIZE", "Counter_Value": 70.0},
    ]
    write_csv(str(tmp_path / "fetch" / "x_counter_collection.csv"), fields, fetch_rows)
    write_csv(str(tmp_path / "write" / "x_counter_collection.csv"), fields, write_rows)
    return str(kt), str(tmp_path / "fetch"), str(tmp_path / "write")


def test_summary_scales_by_copy_calibration(tmp_path, monkeypatch):
    bench = load_bench(tmp_path, monkeypatch)
    bench.summarize_prof(*fake_profiles(tmp_path))
    # copy: FETCH reads half of the 1 GiB it moved -> scale 2; WRITE exact -> scale 1
    # extend: (mean fetch 200 KiB * 2 + 10 KiB) per dispatch
    assert bench.measured_traffic("extend") == (200 * 2 + 10) * 1024
    assert bench.measured_traffic("decode") == (50 * 2 + 70) * 1024
    text = open(bench.TRAFFIC_FILE).read()
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text


def test_stale_summary_is_ignored(tmp_path, monkeypatch):
    bench = load_bench(tmp_path, monkeypatch)
    bench.summarize_prof(*fake_profiles(tmp_path))
    real = bench.source_sha
    monkeypatch.setattr(bench, "source_sha", lambda kind: "0" * 64 if kind == "extend" else real(kind))
    assert bench.measured_traffic("extend") is None
    assert bench.measured_traffic("decode") is not None


def test_missing_summary_gives_none(tmp_path, monkeypatch):
    bench = load_bench(tmp_path, monkeypatch)
    assert bench.measured_traffic("extend") is None


def test_multi_gpu_request_exits(monkeypatch, capsys):
    import subprocess, sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_runs_the_oracle_over_workers(tmp_path, monkeypatch):
    """The CPU baseline splits the prefill workload into (sequence, head-block) units
    over forked single-threaded workers and reports tokens/s, the workers used, the
    host's CPU count and the one-thread rate."""
    bench = load_bench(tmp_path, monkeypatch)
    res = bench.cpu_baseline(nseq=2, seqlen=16, workers=4)
    assert res["kind"] == "oracle" and res["unit"] == "tokens/s"
    assert res["cores"] == 4 and res["host_cpus"] == os.cpu_count()
    assert res["value"] > 0 and res["one_thread_value"] > 0
    assert "4 (sequence, 16-head) units" in res["sample"]
    assert 1 <= bench.cpu_workers() <= 16



def test_ssd_counter_summary(tmp_path, monkeypatch):
    """The delta-off counter summary: copy-scaled traffic per kernel, their sum against
    the call's algorithmic bytes, and the SQ ratios of each kernel."""
    bench = load_bench(tmp_path, monkeypatch)
    monkeypatch.setattr(bench, "SSD_COUNTERS_FILE", str(tmp_path / "profiles" / "ssd.txt"))
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    copy = "vectorized_elementwise_kernel<MulFunctor<float>>"
    names = {"prep": "gdn::ssd_prep_kernel(gdn::SeqLaunch)",
             "state": "void gdn::ssd_kernel<unsigned short, true, false, false>(gdn::SeqLaunch)",
             "full": "void gdn::ssd_kernel<unsigned short, true, true, false>(gdn::SeqLaunch)"}
    fk = {"prep": 10.0, "state": 20.0, "full": 30.0}
    wk = {"prep": 1.0, "state": 2.0, "full": 3.0}
    write_csv(str(tmp_path / "f" / "a_counter_collection.csv"), fields,
              [{"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 524288.0}] +
              [{"Kernel_Name": names[k], "Counter_Name": "FETCH_SIZE", "Counter_Value": v} for k, v in fk.items()])
    write_csv(str(tmp_path / "w" / "a_counter_collection.csv"), fields,
              [{"Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1048576.0}] +
              [{"Kernel_Name": names[k], "Counter_Name": "WRITE_SIZE", "Counter_Value": v} for k, v in wk.items()])
    sq1 = [{"Kernel_Name": names["full"], "Counter_Name": c, "Counter_Value": v}
           for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 40.0), ("SQ_BUSY_CU_CYCLES", 100.0),
                        ("SQ_INSTS_MFMA", 10.0), ("SQ_INSTS_VALU", 35.0))]
    sq2 = [{"Kernel_Name": names["full"], "Counter_Name": "SQ_WAIT_ANY", "Counter_Value": 5.0}]
    write_csv(str(tmp_path / "s1" / "a_counter_collection.csv"), fields, sq1)
    write_csv(str(tmp_path / "s2" / "a_counter_collection.csv"), fields, sq2)
    bench.summarize_ssd_counters(*(str(tmp_path / d) for d in ("f", "w", "s1", "s2")))
    kv = {}
    for line in open(bench.SSD_COUNTERS_FILE).read().splitlines():
        if line and not line.startswith("#") and len(line.split()) == 2:
            kv[line.split()[0]] = line.split()[1]
    assert int(kv["full_pass_traffic_bytes"]) == (30 * 2 + 3) * 1024
    assert int(kv["call_traffic_bytes"]) == ((10 + 20 + 30) * 2 + 1 + 2 + 3) * 1024
    assert int(kv["call_algorithmic_bytes"]) == 2 * 8192 * bench.SSD_BYTES_PER_TOKEN + 2 * 80 * 64 * 128 * 4
    text = open(bench.SSD_COUNTERS_FILE).read()
    assert "MFMA busy cycles / (busy CU cycles x 4 SIMDs): 0.100" in text
    assert "VALU instructions per MFMA instruction: 3.5" in text

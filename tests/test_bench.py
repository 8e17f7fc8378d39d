"""CPU checks of bench.py's contract pieces: the multi-GPU refusal and the
counter-to-traffic arithmetic (no GPU needed)."""
from __future__ import annotations

import csv
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_weight_bytes_formula():
    b = _bench()
    # decode_gate_up: 34816 rows of 5120 codes (2560 B) and 160 fp16 scales (320 B)
    assert b.weight_bytes(34816, 5120) == 34816 * (2560 + 320) == 100270080


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "1_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_pmc_scales_by_the_copy(tmp_path):
    b = _bench()
    mib = 256
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    # the copy reads 256 MiB but FETCH_SIZE shows half; WRITE_SIZE shows all
    _write_counters(fetch, [
        {"Kernel_Name": "neg_kernel", "Counter_Name": "FETCH_SIZE", "Counter_Value": mib * 512},
        {"Kernel_Name": "q4::gemv_lds_kernel<1,2,1>", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 1000.0},
        {"Kernel_Name": "q4::gemv_lds_kernel<1,2,1>", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 1002.0},
    ])
    _write_counters(write, [
        {"Kernel_Name": "neg_kernel", "Counter_Name": "WRITE_SIZE", "Counter_Value": mib * 1024},
        {"Kernel_Name": "q4::gemv_lds_kernel<1,2,1>", "Counter_Name": "WRITE_SIZE",
         "Counter_Value": 10.0},
    ])
    out = str(tmp_path / "rec.json")
    b.summarize_pmc(fetch, write, mib, "t", "gemv_lds_kernel", 2_000_000, out)
    rec = json.load(open(out))
    assert rec["calibration"]["read_factor"] == 2.0
    assert rec["calibration"]["write_factor"] == 1.0
    assert rec["hbm_bytes_per_launch"] == round(1001.0 * 1024 * 2 + 10.0 * 1024)
    assert rec["dispatches"] == {"FETCH_SIZE": 2, "WRITE_SIZE": 1}


def test_traffic_record_is_ignored_for_other_sources(tmp_path, monkeypatch):
    b = _bench()
    d = tmp_path / "profiles"
    d.mkdir()
    (d / "k_pmc.json").write_text(json.dumps({"csrc_digest": "old", "hbm_bytes_per_launch": 5}))
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.traffic_from_profile("k", "new") is None
    assert b.traffic_from_profile("k", "old") == 5


def test_summarize_trace_percentiles(tmp_path):
    b = _bench()
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    with open(d / "7_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        # kernel a: 1..10 us; kernel b: one 100 us launch
        for i in range(1, 11):
            w.writerow({"Kernel_Name": "void q4::a<1>(int)", "Start_Timestamp": 1000 * i,
                        "End_Timestamp": 1000 * i + 1000 * i})
        w.writerow({"Kernel_Name": "void q4::(anonymous namespace)::b<2>(float*)",
                    "Start_Timestamp": 0, "End_Timestamp": 100000})
    s = b.summarize_trace(str(tmp_path / "trace"))
    assert list(s) == ["q4::b<2>", "q4::a<1>"]       # by total time
    a = s["q4::a<1>"]
    assert a["calls"] == 10 and a["mean_us"] == 5.5 and a["median_us"] == 5.5
    assert a["p10_us"] == 1.9 and a["p90_us"] == 9.1
    assert a["min_us"] == 1.0 and a["max_us"] == 10.0
    assert s["q4::b<2>"]["calls"] == 1 and s["q4::b<2>"]["median_us"] == 100.0


def test_summarize_counters_means(tmp_path):
    b = _bench()
    d = tmp_path / "pmc" / "host"
    d.mkdir(parents=True)
    with open(d / "9_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        # kernel a: two dispatches of two counters; kernel b: one dispatch
        for v in (10.0, 30.0):
            w.writerow({"Kernel_Name": "void q4::a<1>(int)", "Counter_Name": "SQ_WAVES",
                        "Counter_Value": v})
            w.writerow({"Kernel_Name": "void q4::a<1>(int)", "Counter_Name": "FETCH_SIZE",
                        "Counter_Value": 2 * v})
        w.writerow({"Kernel_Name": "void q4::(anonymous namespace)::b<2>(float*)",
                    "Counter_Name": "SQ_WAVES", "Counter_Value": 7})
    s = b.summarize_counters([str(tmp_path / "pmc")])
    assert s["q4::a<1>"] == {"dispatches": {"FETCH_SIZE": 2, "SQ_WAVES": 2},
                             "FETCH_SIZE": 40.0, "SQ_WAVES": 20.0}
    assert s["q4::b<2>"] == {"dispatches": {"SQ_WAVES": 1}, "SQ_WAVES": 7.0}


def test_counters_table_derived_figures(tmp_path):
    """The text table: per-wave VALU, MFMA busy fraction and calibrated MB,
    from passes in separate run folders."""
    b = _bench()
    runs = []
    rows = {"sq": [("SQ_WAVES", 64.0), ("SQ_INSTS_VALU", 6400.0), ("SQ_INSTS_MFMA", 3.0),
                   ("SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 50), ("GRBM_GUI_ACTIVE", 8.0 * 100)],
            "fetch": [("FETCH_SIZE", 1000.0)], "write": [("WRITE_SIZE", 500.0)]}
    neg = {"fetch": ("FETCH_SIZE", 256 * 1024 / 2), "write": ("WRITE_SIZE", 256 * 1024)}
    for run, cs in rows.items():
        d = tmp_path / run / "host"
        d.mkdir(parents=True)
        with open(d / "1_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for c, v in cs:
                w.writerow({"Kernel_Name": "void q4::k(int)", "Counter_Name": c,
                            "Counter_Value": v})
            if run in neg:
                w.writerow({"Kernel_Name": "void at::native::neg_kernel_x(int)",
                            "Counter_Name": neg[run][0], "Counter_Value": neg[run][1]})
        runs.append(str(tmp_path / run))
    text = b.counters_table(b.summarize_counters(runs))
    line = [l for l in text.splitlines() if l.startswith("q4::k")][0].split()
    # waves, VALU/wave, MFMA, busy %, LDS/wave (absent), bank cf (absent), MB read, MB written
    assert line[1:5] == ["64", "100", "3", "50.0%"]
    assert float(line[-2]) == round(1000 * 1024 * 2 / 1e6, 1)
    assert float(line[-1]) == round(500 * 1024 / 1e6, 2)


def test_build_records_its_commit(tmp_path, monkeypatch):
    spec = importlib.util.spec_from_file_location(
        "q4_build", os.path.join(ROOT, "quantized_q4_block_amd", "_build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    info = b._build_info()
    assert set(info) == {"commit", "sources_modified"}
    if info["commit"] is not None:    # a git checkout
        assert len(info["commit"]) == 40 and isinstance(info["sources_modified"], bool)
    # bench reads the record the build wrote, and copes with its absence
    bench = _bench()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.library_build_info() is None
    (tmp_path / "quantized_q4_block_amd").mkdir()
    (tmp_path / "quantized_q4_block_amd" / "build_info.json").write_text(
        '{"commit": "abc", "sources_modified": true}')
    assert bench.library_build_info() == {"commit": "abc", "sources_modified": True}

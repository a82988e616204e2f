"""Host logic of bench.py (no GPU): the one-GPU contract and the counter
summary that decides whether the bench line carries an HBM traffic figure."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for did, name, value in rows:
            w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_counter_summary_scales_by_the_calibrators_and_tracks_the_sources(tmp_path):
    cal_kib = bench.CAL_BYTES / 1024.0
    # the read probe (decode-shaped loads) reads as half its bytes in FETCH_SIZE
    # (two launches, grid-strided and blocked); the fill kernel writes all of its
    fetch = [(1, "k_stream_read<8, true>", cal_kib / 2), (2, "k_stream_read<8, true>", cal_kib / 2),
             (3, "k_zero", 0.0), (4, "k_decode_mfma<128,4,4>", 1000.0),
             (5, "k_decode_mfma<128,4,4>", 1002.0)]
    write = [(1, "k_stream_read<8, true>", 0.0), (2, "k_stream_read<8, true>", 0.0),
             (3, "k_zero", cal_kib), (4, "k_decode_mfma<128,4,4>", 10.0),
             (5, "k_decode_mfma<128,4,4>", 10.0)]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    recs = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                    "llama8b-512k", str(out))
    key = "k_decode_mfma@llama8b-512k"
    expect = round(1001.0 * 1024 * 2 + 10.0 * 1024)
    assert recs[key]["hbm_bytes_per_launch"] == expect
    assert recs[key]["calibration"]["FETCH_SIZE"]["scale"] == 2.0
    assert bench.traffic_record("k_decode_mfma", "llama8b-512k", str(out)) == expect
    # a second workload is merged in beside the first
    bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "llama8b-128k",
                             str(out))
    assert bench.traffic_record("k_decode_mfma", "llama8b-128k", str(out)) == expect
    assert bench.traffic_record("k_decode_mfma", "llama8b-512k", str(out)) == expect
    # counters taken on other kernel sources are not reported
    stale = json.loads(out.read_text())
    stale[key]["sources"] = "0" * 16
    out.write_text(json.dumps(stale))
    assert bench.traffic_record("k_decode_mfma", "llama8b-512k", str(out)) is None
    assert bench.traffic_record("k_decode_valu", "llama8b-512k", str(out)) is None


def test_cpu_baseline_is_the_oracle_on_the_active_groups():
    # A small layer through the CPU-baseline leg: its pieces merged per group
    # equal the oracle's attention of each group, and the report names the
    # threads it used.
    import numpy as np

    import oracle
    from workloads import Workload, as_numpy, make_layer
    wl = Workload("cpu-small", 1, 8, 2, 64, 3000, "bf16", seed=5, sink_plan=("count", 1))
    layer = make_layer(wl)
    q_np, k_np, v_np = as_numpy(layer.q), as_numpy(layer.k), as_numpy(layer.v)
    ref = oracle.dense_decode(q_np, k_np, v_np)
    slabs = {j: (q_np[0, 4 * j:4 * j + 4], k_np[0, j], v_np[0, j]) for j in (0, 1)}
    rep = bench.cpu_baseline(wl, q_np, k_np[:, :, 0], slabs, 0.5, budget_s=0.05, chunk=512,
                             gpu_out=ref.astype(np.float32))
    assert rep["kind"] == "oracle" and rep["cores"] >= 1 and rep["passes"] >= 1
    assert rep["max_abs_vs_gpu"] < 1e-6  # the fp32 rounding of the reference only


def test_source_digest_ignores_comments_only():
    code = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    assert bench._code_only(code) == bench._code_only(code.replace("one more", "the next"))
    assert bench._code_only(code) == bench._code_only("/* doc */ int f(int x){return x+1;}")
    assert bench._code_only(code) != bench._code_only(code.replace("x + 1", "x + 2"))

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


def test_counter_summary_scales_by_the_copy_and_tracks_the_sources(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024.0
    # the copy reads as half its bytes in FETCH_SIZE and all of them in WRITE_SIZE
    fetch = [(1, "__amd_rocclr_copyBuffer", copy_kib / 2), (2, "k_decode_mfma<128,4,4>", 1000.0),
             (3, "k_decode_mfma<128,4,4>", 1002.0)]
    write = [(1, "__amd_rocclr_copyBuffer", copy_kib), (2, "k_decode_mfma<128,4,4>", 10.0),
             (3, "k_decode_mfma<128,4,4>", 10.0)]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    recs = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out))
    key = "k_decode_mfma@llama8b-512k"
    expect = round(1001.0 * 1024 * 2 + 10.0 * 1024)
    assert recs[key]["hbm_bytes_per_launch"] == expect
    assert bench.traffic_record("k_decode_mfma", "llama8b-512k", str(out)) == expect
    # counters taken on other kernel sources are not reported
    stale = json.loads(out.read_text())
    stale[key]["sources"] = "0" * 16
    out.write_text(json.dumps(stale))
    assert bench.traffic_record("k_decode_mfma", "llama8b-512k", str(out)) is None
    assert bench.traffic_record("k_decode_valu", "llama8b-512k", str(out)) is None


def test_source_digest_ignores_comments_only():
    code = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    assert bench._code_only(code) == bench._code_only(code.replace("one more", "the next"))
    assert bench._code_only(code) == bench._code_only("/* doc */ int f(int x){return x+1;}")
    assert bench._code_only(code) != bench._code_only(code.replace("x + 1", "x + 2"))

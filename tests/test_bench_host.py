"""Host-side logic of bench.py (no GPU): the algorithmic byte count the
reported bandwidth divides by, the single-GPU guard, the source hash that
marks counter figures stale, and the scaling of the HBM counters."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_1m_token_layer():
    # 8 KV heads x 65,536 pages x 776 B of record payload + 4 B of page table
    # per page; 1024 selected page-heads x 8 KiB of bf16 K+V, q and output in
    # fp32 for 32 heads, 4 B per selected id (128 per KV head)
    score, attn = bench.algorithmic_bytes(1, 32, 8, 65536, 128, 1024)
    assert score == 8 * 65536 * 776 + 65536 * 4 == 407_109_632
    assert attn == 1024 * 8192 + 32 * 128 * 4 * 2 + 8 * 128 * 4
    assert score + attn == 415_535_104


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()


def test_source_hash_ignores_comments_and_whitespace(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) { return x + 1; }  // one\n")
    b.write_text("/* block\n comment */\nint  f(int x)\n{\n  return x + 1;\n}\n// other words\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_hash([str(a)]) == bench.source_hash([str(b)])
    assert bench.source_hash([str(a)]) != bench.source_hash([str(c)])


def _counter_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": "X",
                        "Counter_Value": value})


def test_traffic_scaling_uses_the_plain_scorer_and_the_last_copies(tmp_path, monkeypatch):
    plain = "void locks::(anonymous namespace)::score_kernel<4, 64, false>(locks::(anonymous namespace)::ScoreArgs)"
    filling = plain.replace("false", "true")
    exact = "void locks::(anonymous namespace)::exact_score_kernel<4>(locks::(anonymous namespace)::ExactArgs)"
    copy = "__amd_rocclr_copyBuffer"
    # an early copy (input upload) is ignored; the last three are the calibration
    fetch_rows = [(copy, 5.0), (plain, 1000.0), (filling, 9999.0), (exact, 7777.0), (plain, 1200.0),
                  (copy, 131000.0), (copy, 131072.0), (copy, 131100.0)]
    write_rows = [(copy, 5.0), (plain, 40.0), (filling, 999.0), (plain, 60.0),
                  (copy, 262144.0), (copy, 262144.0), (copy, 262144.0)]
    fcsv, wcsv, log = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "bench.log"
    _counter_csv(fcsv, fetch_rows)
    _counter_csv(wcsv, write_rows)
    log.write_text("[bench] workload note\n" + json.dumps(
        {"config": {"workload": "synthetic test workload"},
         "roofline": {"algorithmic_bytes_per_launch": 123456}}) + "\n")
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(out))
    bench.traffic_from(str(fcsv), str(wcsv), str(log))
    t = json.loads(out.read_text())
    # per dispatch of the plain scorer: fetch 1100 KiB, write 50 KiB; the
    # median calibration copy reads 131072 KiB fetched (x2.0) and 262144 KiB
    # written (x1.0) for 256 MiB copied
    assert t["fetch_kib_per_dispatch_raw"] == pytest.approx(1100.0)
    assert t["write_kib_per_dispatch_raw"] == pytest.approx(50.0)
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["hbm_bytes_per_launch"] == int(1100.0 * 2.0 * 1024 + 50.0 * 1.0 * 1024)
    assert t["algorithmic_bytes_per_launch"] == 123456
    assert t["workload"] == "synthetic test workload"
    assert t["kernel_source_sha256"] == bench.source_hash(bench.SCORE_SOURCES)

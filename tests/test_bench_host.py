"""Host-side checks of bench.py: argument handling, the useful-work count and
the rule that measured HBM traffic is reported only for the kernel source,
workload and rank it was taken on.  No GPU is used."""

import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle.attention import useful_pairs  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_exits_with_a_message():
    p = _run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU only" in p.stderr and p.stdout == ""


def test_unknown_workload_exits_with_a_message():
    p = _run("--workload", "no_such_workload")
    assert p.returncode == 2
    assert "unknown workload" in p.stderr and p.stdout == ""


def test_head_options_only_for_allgather_workloads():
    p = _run("--workload", "gqa_cp2_s8192", "--kv-heads", "2")
    assert p.returncode == 2
    assert "AllGather-KV" in p.stderr and p.stdout == ""


@pytest.mark.parametrize("q_len,kv_len", [(1, 1), (5, 5), (7, 19), (64, 256), (300, 1000)])
def test_causal_pairs_closed_form_matches_count(q_len, kv_len):
    assert bench.causal_pairs(q_len, kv_len) == useful_pairs(q_len, kv_len, True)


def test_causal_pairs_of_the_long_share():
    # cp 8, blocks b = 8192, rank 3: halves (b, 4b) and (b, 13b); equal blocks
    # give b^2 (2cp - 1) + b (b + 1) pairs per head on every rank
    b = 8192
    total = bench.causal_pairs(b, 4 * b) + bench.causal_pairs(b, 13 * b)
    assert total == b * b * 15 + b * (b + 1) == 1073750016


def test_traffic_reported_only_for_its_source_workload_and_rank(tmp_path, monkeypatch):
    src = tmp_path / "k.h"
    src.write_text("kernel source")
    inc = tmp_path / "tables.h"
    inc.write_text("tables")
    sha = hashlib.sha256(b"kernel sourcetables").hexdigest()
    rec = {"workload": "long_cp8_s131072_r3", "rank": 3,
           "kernels": {"attn_kernel": {"kernel_sha256": sha, "bytes_per_launch": 123}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_PATH", str(path))
    monkeypatch.setitem(bench.KERNEL_SRC, "attn_kernel", [str(src), str(inc)])
    assert bench.traffic_for("attn_kernel", "long_cp8_s131072_r3", 3) == 123
    assert bench.traffic_for("attn_kernel", "long_cp8_s131072_r3", 2) is None
    assert bench.traffic_for("attn_kernel", "gqa_cp2_s8192", 3) is None
    assert bench.traffic_for("scatter_kernel", "long_cp8_s131072_r3", 3) is None   # not recorded
    src.write_text("kernel source, changed")
    assert bench.traffic_for("attn_kernel", "long_cp8_s131072_r3", 3) is None


def _counter_csv(path, rows):
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writerows(rows)


def test_record_traffic_scales_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    """Four rocprofv3 --pmc CSVs -> bytes per launch = FETCH_SIZE * (1 GiB /
    copy FETCH_SIZE) + WRITE_SIZE * (1 GiB / copy WRITE_SIZE), per kernel,
    averaged over dispatches, each record stamped with its source hash."""
    kib = 1 << 20
    _counter_csv(tmp_path / "f" / "x" / "run_counter_collection.csv",
                 [(1, "void cpattn::attn_kernel<128, 1>(A)", "FETCH_SIZE", 1000.0),
                  (2, "void cpattn::attn_kernel<128, 1>(A)", "FETCH_SIZE", 3000.0),
                  (3, "cpattn::rerange_kernel(...)", "FETCH_SIZE", 500.0),
                  (4, "cpattn::scatter_kernel(...)", "FETCH_SIZE", 700.0)])
    _counter_csv(tmp_path / "w" / "run_counter_collection.csv",
                 [(1, "void cpattn::attn_kernel<128, 1>(A)", "WRITE_SIZE", 100.0),
                  (3, "cpattn::rerange_kernel(...)", "WRITE_SIZE", 400.0),
                  (4, "cpattn::scatter_kernel(...)", "WRITE_SIZE", 800.0)])
    _counter_csv(tmp_path / "cf" / "run_counter_collection.csv",
                 [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2)])
    _counter_csv(tmp_path / "cw" / "run_counter_collection.csv",
                 [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", kib)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_PATH", str(out))
    bench.record_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                         str(tmp_path / "cw"), "long_cp8_s131072_r3", 3)
    rec = json.loads(out.read_text())
    assert rec["copy_calibration"]["fetch_factor"] == 2.0 and rec["copy_calibration"]["write_factor"] == 1.0
    k = rec["kernels"]
    assert k["attn_kernel"]["bytes_per_launch"] == (2000.0 * 2 + 100.0) * 1024
    assert k["rerange_kernel"]["bytes_per_launch"] == (500.0 * 2 + 400.0) * 1024
    assert k["scatter_kernel"]["bytes_per_launch"] == (700.0 * 2 + 800.0) * 1024
    assert k["attn_kernel"]["kernel_sha256"] == bench.kernel_sha256(bench.KERNEL_SRC["attn_kernel"])

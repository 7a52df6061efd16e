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
    (tmp_path / "profiles").mkdir()
    rec = {"kernel_sha256": sha, "workload": "long_cp8_s131072_r3", "rank": 3, "bytes_per_launch": 123}
    (tmp_path / "profiles" / "attn_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for([str(src), str(inc)], "long_cp8_s131072_r3", 3) == 123
    assert bench.traffic_for([str(src), str(inc)], "long_cp8_s131072_r3", 2) is None
    assert bench.traffic_for([str(src), str(inc)], "gqa_cp2_s8192", 3) is None
    src.write_text("kernel source, changed")
    assert bench.traffic_for([str(src), str(inc)], "long_cp8_s131072_r3", 3) is None

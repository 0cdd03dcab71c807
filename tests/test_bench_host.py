"""Host logic of bench.py that runs without a GPU: the one-GPU guard, and the
rule that counter-derived traffic is reported only while the batched decode
kernel's source it was taken on is unchanged (whole-line comments aside)."""
from __future__ import annotations

import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _copy_tree(tmp_path):
    dst = tmp_path / "mixed_precision_weight_dq_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "mixed_precision_weight_dq_amd", "csrc"), dst)
    return dst


def test_digest_ignores_comment_lines_only(tmp_path, monkeypatch):
    csrc = _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_digest()
    gemv = csrc / "gemv_batch.hip"
    text = gemv.read_text()
    gemv.write_text("// a comment line\n" + text)
    assert bench.kernel_source_digest() == base
    gemv.write_text(text.replace("namespace dq {", "namespace dq {\nconstexpr int kUnused = 1;", 1))
    assert bench.kernel_source_digest() != base


def test_recorded_traffic_only_for_the_current_source(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.recorded_traffic() is None  # no file
    rec.write_text(json.dumps({"source_digest": bench.kernel_source_digest(),
                               "bytes_per_launch_avg": 1234}))
    assert bench.recorded_traffic() == 1234
    rec.write_text(json.dumps({"source_digest": "0" * 16, "bytes_per_launch_avg": 1234}))
    assert bench.recorded_traffic() is None
    rec.write_text("not json")
    assert bench.recorded_traffic() is None

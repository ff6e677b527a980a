"""bench.py's host-side contract (no GPU): the one-GPU guard, the workload
labels, and the rule that HBM traffic from a counter summary is reported
only while the kernel sources still hash to the digest recorded with it."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_workload_labels_cover_every_workload():
    assert set(bench.WORKLOADS.values()) == {0, 1, 2, 3, 4}
    assert set(synth.WORKLOAD_NAMES) == {0, 1, 2, 3, 4}
    assert bench.WORKLOADS["c1"] == 1


def _fake_tree(tmp_path, body):
    csrc = tmp_path / "mqa_logits_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text(body)
    (csrc / "b.hpp").write_text("// header\n")
    (tmp_path / "profiles").mkdir()
    return tmp_path


def _summary(root, digest, total="123456"):
    (root / "profiles" / "k_w1_traffic.txt").write_text(
        "# comment: lines starting with # are ignored\n"
        "kernel: k\n"
        "sources: a.hip b.hpp\n"
        f"source_sha256: {digest}\n"
        f"hbm_bytes_per_launch: {total}\n")


def test_traffic_is_reported_for_matching_sources(tmp_path, monkeypatch):
    root = _fake_tree(tmp_path, "kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    _summary(root, bench.kernel_source_digest(["a.hip", "b.hpp"]))
    assert bench.measured_traffic("w1") == pytest.approx(123456.0)
    assert bench.measured_traffic("w2") is None          # no summary for that workload


def test_traffic_is_dropped_once_a_source_changes(tmp_path, monkeypatch):
    root = _fake_tree(tmp_path, "kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    _summary(root, bench.kernel_source_digest(["a.hip", "b.hpp"]))
    (root / "mqa_logits_amd" / "csrc" / "a.hip").write_text("kernel v2\n")
    assert bench.measured_traffic("w1") is None


def test_traffic_is_dropped_when_a_listed_source_is_missing(tmp_path, monkeypatch):
    root = _fake_tree(tmp_path, "kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    _summary(root, bench.kernel_source_digest(["a.hip", "b.hpp"]))
    os.remove(root / "mqa_logits_amd" / "csrc" / "b.hpp")
    assert bench.measured_traffic("w1") is None


def test_digest_depends_on_names_and_contents(tmp_path, monkeypatch):
    root = _fake_tree(tmp_path, "kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    d1 = bench.kernel_source_digest(["a.hip", "b.hpp"])
    assert d1 == bench.kernel_source_digest(["b.hpp", "a.hip"])   # order-free
    assert d1 != bench.kernel_source_digest(["a.hip"])

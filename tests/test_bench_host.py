"""Host logic of bench.py that needs no GPU: the HBM traffic figure it
reports from the committed counter summaries, and the one-GPU guard."""

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synthetic as S  # noqa: E402


def test_committed_traffic_record_matches_the_committed_kernel():
    # the decode counters were taken on the kernel source as committed; a
    # record left behind by a later change would report no traffic at all
    t = bench.recorded_traffic("gateup_fused_kernel", "decode")
    assert isinstance(t, int)
    # within 3 % of the launch's algorithmic bytes (the whole one-token
    # layer with 6 routed experts, 135.98 MB). The excess allowed covers the
    # down workgroups' reads of the h rows as 8-byte words; one expert's
    # down matrix (6.2 MB, 4.6 %) read twice would exceed it.
    _, algo = bench.kernel_work("gateup_fused_kernel", S.get("decode"), 6)
    assert abs(algo / 135.98e6 - 1.0) < 1e-4
    assert abs(t / algo - 1.0) < 0.03


def _fake_tree(tmp_path, src_text, recorded_sha):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text(src_text)
    (tmp_path / "profiles" / "k_traffic.md").write_text(
        "kernel: some_kernel\nworkload: w\ntraffic_bytes_per_launch: 1234\n"
        f"kernel_source: k.hip\nkernel_source_sha256: {recorded_sha}\n")


def test_traffic_is_reported_only_while_the_source_is_unchanged(tmp_path, monkeypatch):
    src = "__global__ void some_kernel() {}\n"
    _fake_tree(tmp_path, src, hashlib.sha256(src.encode()).hexdigest())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("some_kernel", "w") == 1234
    assert bench.recorded_traffic("some_kernel", "other") is None
    assert bench.recorded_traffic("other_kernel", "w") is None
    (tmp_path / "k.hip").write_text(src + "// edited\n")
    assert bench.recorded_traffic("some_kernel", "w") is None


def test_traffic_without_its_source_file_is_not_reported(tmp_path, monkeypatch):
    _fake_tree(tmp_path, "x", "0" * 64)
    os.remove(tmp_path / "k.hip")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("some_kernel", "w") is None


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "--gpus 1" in (r.stdout + r.stderr)

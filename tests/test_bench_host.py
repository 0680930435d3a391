"""Host logic of bench.py (no GPU): the traffic summaries' parsing and their
tie to the GEMM sources, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_summary(tmp_path, sha, fetch_kib, write_kib, copy_fetch_kib, copy_write_kib):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / f"k_gemm8_{bench.SLUG['c5']}_traffic.txt").write_text(
        "# a summary\n"
        f"gemm_source_sha256 = {sha}\n"
        f"fetch_kib = {fetch_kib}\n"
        f"write_kib = {write_kib}\n"
        f"copy_fetch_kib = {copy_fetch_kib}\n"
        f"copy_write_kib = {copy_write_kib}\n")


def test_traffic_scales_counters_by_the_copy(tmp_path, monkeypatch):
    # the copy of COPY_BYTES reads FETCH 1/2 and WRITE 1 KiB per true KiB:
    # a GEMM counter reading of F and W KiB means 2F and W KiB of traffic
    copy_kib = bench.COPY_BYTES / 1024
    _write_summary(tmp_path, bench.gemm_source_sha256(), 1000.0, 300.0, copy_kib / 2, copy_kib)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_per_launch("c5") == pytest.approx((2 * 1000.0 + 300.0) * 1024)


def test_traffic_is_null_for_other_gemm_sources(tmp_path, monkeypatch):
    copy_kib = bench.COPY_BYTES / 1024
    _write_summary(tmp_path, "0" * 64, 1000.0, 300.0, copy_kib / 2, copy_kib)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_per_launch("c5") is None


def test_traffic_is_null_without_a_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_per_launch("c5") is None


def test_committed_summaries_parse():
    # every committed summary names a source hash and the four counters
    for key, slug in bench.SLUG.items():
        path = os.path.join(ROOT, "profiles", f"k_gemm8_{slug}_traffic.txt")
        if not os.path.exists(path):
            continue
        kv = dict(line.split("=", 1) for line in open(path) if "=" in line)
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        assert len(kv["gemm_source_sha256"]) == 64, key
        for k in ("fetch_kib", "write_kib", "copy_fetch_kib", "copy_write_kib"):
            assert float(kv[k]) > 0, (key, k)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr

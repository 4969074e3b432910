"""Host logic of bench.py (no GPU): the readers that take the measured HBM traffic and the kernel
durations of a profiled unit from rocprofv3 summaries, and refuse them once the library sources
differ from those the summaries were taken on."""
from __future__ import annotations

import os

import pytest

import bench


@pytest.fixture
def root(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha256", lambda: "abc123")
    return tmp_path


def _trace(sha: str) -> str:
    head = ["# rocprofv3 kernel trace + stats, test", "# command: ...",
            f"# library sources sha256 (clustered_retrieval_lm_amd/csrc/*): {sha}", "# durations in microseconds",
            f"{'kernel':78s} {'calls':>6s} {'total_us':>11s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s} {'pct':>6s}"]
    rows = [("void fh::k_b1_stage2<1, 3, 4, 2>(fh::B1Params)", 8780, 10.126),
            ("void fh::k_mfma<4, 4, 1>(fh::MfmaParams)", 140, 152.5),      # the dense comparator's
            ("void fh::k_mfma<4, 3, 0>(fh::MfmaParams)", 9024, 14.0),     # the head's: launched most
            ("void fh::k_finalize_parts<1>(unsigned long const*, int, int*)", 8780, 4.009)]
    body = [f"{n:78s} {c:6d} {c * a:11.1f} {a:8.3f} {a / 2:8.3f} {a * 2:8.3f} {10.0:6.2f}" for n, c, a in rows]
    return "\n".join(head + body) + "\n"


def test_profiled_us_reads_the_head_kernels(root):
    (root / "profiles" / "kernel_trace_w_b1.txt").write_text(_trace("abc123"))
    got = bench.profiled_us("w_b1", ["fh::k_b1_stage2", "fh::k_finalize_parts", "fh::k_mfma", "fh::k_absent"])
    assert got == {"fh::k_b1_stage2": 10.126, "fh::k_finalize_parts": 4.009, "fh::k_mfma": 14.0}


def test_profiled_us_refuses_other_sources_and_missing_files(root):
    (root / "profiles" / "kernel_trace_w_b1.txt").write_text(_trace("other"))
    assert bench.profiled_us("w_b1", ["fh::k_b1_stage2"]) is None
    assert bench.profiled_us("none_b1", ["fh::k_b1_stage2"]) is None


def test_measured_traffic_sums_the_unit_and_checks_the_sources(root):
    text = ("source_sha256: abc123\nfetch_factor: 2.0000\nwrite_factor: 1.0000\n"
            "kernel: fh::k_b1_stage2<1,3,4,2> dispatches=10 FETCH_SIZE_KiB=9765.87 WRITE_SIZE_KiB=8.00 traffic_bytes=20008245\n"
            "kernel: fh::k_finalize_parts<1> dispatches=10 FETCH_SIZE_KiB=2.06 WRITE_SIZE_KiB=0.03 traffic_bytes=4256\n")
    (root / "profiles" / "hbm_traffic_w_b1.txt").write_text(text)
    assert bench.measured_traffic("w_b1", ["fh::k_b1_stage2", "fh::k_finalize_parts"]) == 20008245 + 4256
    assert bench.measured_traffic("w_b1", ["fh::k_b1_stage2", "fh::k_absent"]) is None
    (root / "profiles" / "hbm_traffic_w_b1.txt").write_text(text.replace("abc123", "other"))
    assert bench.measured_traffic("w_b1", ["fh::k_b1_stage2"]) is None

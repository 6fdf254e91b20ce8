"""Host-side pieces of bench.py on the CPU: the roofline's traffic figure is
read from a counter summary only when that summary names the current kernel
source; the CPU model is read from the host; the measured peaks are null
without their library."""

import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _summary(path, sha, nbytes):
    with open(path, "w") as f:
        f.write(f"kernel_source_sha256: {sha}\ntraffic_bytes_per_launch: {nbytes}\n")


def test_traffic_only_for_the_current_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.h"
    src.write_text("// kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    summary = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    assert bench.kernel_traffic() is None                 # no summary
    _summary(summary, sha, 504311031)
    assert bench.kernel_traffic() == 504311031.0          # matching source
    src.write_text("// kernel source, edited\n")
    assert bench.kernel_traffic() is None                 # stale summary
    summary.write_text("traffic_bytes_per_launch: 1\n")
    assert bench.kernel_traffic() is None                 # no source hash


def test_cpu_model_and_peaks_without_library(monkeypatch, tmp_path):
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)
    monkeypatch.setattr(bench, "PEAKS_LIB", str(tmp_path / "missing.so"))
    assert bench.measured_peaks(None, None) is None


def test_attn_flops():
    assert bench.attn_flops(1, 24, 8192, 32768, 128) == 3298534883328

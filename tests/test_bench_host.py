"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
bookkeeping that turns counter summaries into the roofline's traffic."""

from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flop_conventions():
    # forward 4*B*H*S^2*D (half when causal); backward 2.5x the forward
    f = 4.0 * bench.B * bench.H * bench.S * bench.S * bench.D
    assert bench.fwd_flops(False) == f and bench.fwd_flops(True) == f / 2
    assert bench.bwd_flops(False) == 2.5 * f and bench.bwd_flops(True) == 1.25 * f
    # products credited per kernel sum to the five of the backward pass in split mode
    assert bench.KERNEL_PRODUCTS["bwd_dkdv"] + bench.KERNEL_PRODUCTS["bwd_dq"] == bench.KERNEL_PRODUCTS["bwd_main"]


def test_traffic_of_other_sources_is_not_reported(tmp_path, monkeypatch):
    src = open(bench.TRAFFIC_FILES["fwd"]).read()
    stale = tmp_path / "stale.md"
    stale.write_text(src.replace("kernel_source_sha256_16: ", "kernel_source_sha256_16: 0"))
    monkeypatch.setitem(bench.TRAFFIC_FILES, "fwd", str(stale))
    assert bench.read_traffic("fwd") is None
    monkeypatch.setitem(bench.TRAFFIC_FILES, "fwd", str(tmp_path / "missing.md"))
    assert bench.read_traffic("fwd") is None

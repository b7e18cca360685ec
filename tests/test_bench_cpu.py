"""The measurement script's host logic, on the CPU: the one-GPU contract, the
algorithmic byte and flop counts its roofline figures divide by, the choice of
the dominant kernel, and the gating of the counter-measured traffic on the
kernel source it was taken for."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from speculative_decoding_step_amd import configs  # noqa: E402


def test_bench_refuses_several_gpus():
    """--gpus N > 1 exits with a message before touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_verify_work_of_the_8b_tree_step():
    """One batch-1 verify at the 8B shape (61 rows over 2,048 committed positions):
    7.50 B target parameters (32 layers of q, k, v, o, gate, up, down plus the
    128,256 x 4,096 LM head) read once, 15.01 GB in bf16, plus 268 MB of K/V and
    the rows' own K/V and aux: about 15.29 GB; GEMM flops 2 x 61 x 7.50 B."""
    w = configs.WORKLOADS["llama8b_tree_b1"]
    nbytes, flops = bench.verify_work(w)
    assert abs(nbytes - 15.29e9) / 15.29e9 < 2e-3, nbytes
    assert abs(flops - 2 * 61 * 7.504e9) / flops < 1e-3, flops


def test_step_bytes_of_the_8b_tree_step():
    """The whole batch-1 step reads about 24.7 GB: the verify's weights, the six
    draft forwards' layer (243 M parameters) and 1.05 GB head each, the fusion FC,
    and the target and draft K/V."""
    w = configs.WORKLOADS["llama8b_tree_b1"]
    assert abs(bench.step_bytes(w) - 24.7e9) / 24.7e9 < 5e-3, bench.step_bytes(w)


def test_roofline_takes_the_kernel_kind_with_the_most_time():
    """prof[kind] = (launches, ms over the timed steps, algorithmic bytes, flops) for kinds 0, 1, 3:
    the kind with the largest time is reported, HBM-bound for the skinny kernels
    and MFMA-bound for the large-M one, achieved = work / time."""
    w = configs.WORKLOADS["llama8b_tree_b1"]
    # kind 1 has the most time: 6 GB in 2 ms = 3 TB/s, 0.375 of 8 TB/s, 10 launches per step over 2 steps
    r = bench.roofline(w, {0: (10, 1.0, 4e9, 0.0), 1: (20, 2.0, 6e9, 0.0), 3: (0, 0.0, 0.0, 0.0)}, steps=2)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["launches_per_step"] == 10
    assert r["achieved"] == pytest.approx(3000.0) and r["frac"] == pytest.approx(0.375)
    assert r["kernel_ms_per_step"] == pytest.approx(1.0) and r["algorithmic_bytes_per_launch"] == 3e8
    # the large-M kind: 5 TFLOP in 4 ms = 1.25 PFLOP/s, 0.5 of the bf16 peak
    r = bench.roofline(w, {0: (10, 1.0, 1e9, 0.0), 1: (0, 0.0, 0.0, 0.0), 3: (5, 4.0, 0.0, 5e12)}, steps=1)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1250.0) and r["frac"] == pytest.approx(0.5)


def test_measured_traffic_needs_the_same_kernel_source(monkeypatch):
    """The committed counter figure is used only for the kernel kind and source
    digest it was taken for; any other kind, or a changed source, gives None."""
    w = configs.WORKLOADS["llama8b_tree_b1"]
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    with open(path) as f:
        t = json.load(f)
    kind = t["kernel_kind"]
    if t["source_digest"] == bench._kernel_source_digest(kind):
        assert bench.measured_traffic(w, kind) == t["bytes_per_launch"]
    other = 3 if kind != 3 else 0
    assert bench.measured_traffic(w, other) is None
    monkeypatch.setattr(bench, "_kernel_source_digest", lambda k: "0" * 16)
    assert bench.measured_traffic(w, kind) is None

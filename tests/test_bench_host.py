"""Host-side logic of bench.py (no GPU): the algorithmic byte counts behind the roofline
figures, the traffic record and its source check, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

B, T, H, D = 4, 32768, 32, 128
ELEMS = B * T * H * D  # elements of one (batch, seq, heads, dim) tensor at the headline shape
STATE = B * H * D * D * 4  # one fp32 state per (row, head)


def test_forward_bytes_headline():
    # q, k, v in bf16 (2 B each), o in fp32 (4 B), the final state written once
    assert bench.algorithmic_bytes(B, T, H, H, D, D, 2) == ELEMS * (3 * 2 + 4) + STATE == 5_377_097_728
    # a bf16 o halves the output bytes
    assert bench.algorithmic_bytes(B, T, H, H, D, D, 2, o_bytes=2) == ELEMS * (3 * 2 + 2) + STATE
    # an initial state is read as well
    assert bench.algorithmic_bytes(B, T, H, H, D, D, 2, with_init=True) == ELEMS * 10 + 2 * STATE


def test_forward_bytes_gqa_and_dims():
    # kv heads carry k and v; q and o follow the query heads
    got = bench.algorithmic_bytes(1, 100, 8, 2, 64, 32, 2)
    assert got == 100 * (8 * 64 + 2 * 64 + 2 * 32) * 2 + 100 * 8 * 32 * 4 + 8 * 64 * 32 * 4


def test_backward_bytes_headline():
    # q, k, v, dO in (bf16); dq, dk, dv out (fp32); d initial_state out
    assert bench.bwd_algorithmic_bytes(B, T, H, H, D, D, 2) == ELEMS * (4 * 2 + 3 * 4) + STATE == 10_745_806_848


def test_traffic_record_consistent():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    fs = rec["copy_fetch_kib"] * 1024 / rec["copy_probe_bytes"]
    ws = rec["copy_write_kib"] * 1024 / rec["copy_probe_bytes"]
    assert fs == pytest.approx(rec["fetch_scale"], rel=1e-3)
    assert ws == pytest.approx(rec["write_scale"], rel=1e-3)
    fetch = sum(rec["fetch_kib_per_dispatch_raw"]) / len(rec["fetch_kib_per_dispatch_raw"]) * 1024 / rec["fetch_scale"]
    write = sum(rec["write_kib_per_dispatch_raw"]) / len(rec["write_kib_per_dispatch_raw"]) * 1024 / rec["write_scale"]
    assert fetch == pytest.approx(rec["fetch_bytes_per_launch"], rel=1e-6)
    assert write == pytest.approx(rec["write_bytes_per_launch"], rel=1e-6)
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(B, T, H, H, D, D, 2)


def test_traffic_only_for_matching_source(monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "kernel_sha", lambda: rec["kernel_sha"])
    assert bench.measured_traffic() == rec["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0" * 16)
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_ms_stats():
    st = bench.ms_stats([3.0, 1.0, 2.0, 10.0])
    assert st == {"mean": 4.0, "median": 2.5, "min": 1.0, "max": 10.0, "calls": 4}
    assert bench.ms_stats([2.0, 1.0, 5.0])["median"] == 2.0


def test_roofline_pair_bound():
    # the headline at 1.0 ms: 5.38 GB -> 5.38 TB/s (0.67 of HBM); 2.2 TFLOP -> 0.09 of bf16 MFMA
    flops = bench.fwd_algorithmic_flops(B * T, H, D, D)
    assert flops == 4 * B * T * H * D * D
    bound, hbm, mfma = bench.roofline_pair(bench.algorithmic_bytes(B, T, H, H, D, D, 2), flops, 1.0)
    assert bound == "hbm"
    assert hbm["frac"] == pytest.approx(5_377_097_728 / 1e-3 / 1e9 / 8000.0)
    assert mfma["frac"] == pytest.approx(flops / 1e-3 / 1e12 / 2500.0)
    # a compute-heavy kernel names the matrix roofline
    assert bench.roofline_pair(1e6, 1e13, 1.0)[0] == "mfma"


def test_cpu_model_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()

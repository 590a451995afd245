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

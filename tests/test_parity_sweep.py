"""GPU parity over a seeded sweep of small problems that mixes every option at once.

The explicit cases in the other parity files each vary one or two things; here every
case draws its head dims (from the supported pairs of its dtype), batch and head counts,
grouped kv heads, fixed or packed lengths (with empty and one-token sequences), the
direction, an initial state and the layer, so combinations that no explicit case names
are checked too.  Forward for every case and backward for every third, against the
fp64 oracle at the stated bars (both over the whole tensor and per (sequence, head)).
The gated forward gets its own draws: which of the gates g, gk, gv are given, how
strong they are (strong ones send chunks down the exact path), and whether the
Lightning g_gamma is added.
"""
import numpy as np
import pytest

from decayed_recurrent_attention_amd import inputs, lattn
from tests.parity_util import (TOL, check, check_fwd, gpu_run, gpu_run_bwd, gpu_run_gated, oracle_run,
                               oracle_run_bwd, oracle_run_gated)

pytestmark = pytest.mark.gpu

# (dk, dv) pairs the library serves, per input dtype; the backward also runs the kernel
# with the two swapped, so it draws from pairs that are served both ways
DIMS = {
    "bf16": [(32, 16), (32, 48), (64, 64), (64, 112), (128, 32), (128, 96), (128, 128), (192, 64),
             (192, 192), (256, 128)],
    "f32": [(16, 16), (32, 48), (64, 32), (64, 96), (128, 64)],
}
BWD_DIMS = {
    "bf16": [(32, 64), (64, 64), (128, 32), (128, 128), (192, 64), (256, 128)],
    "f32": [(16, 16), (32, 64), (64, 32), (128, 64)],
}
# (dk, dv) pairs of the gated kernels: dk 32, 64, 128 with value blocks of 64 or 16 columns
GATED_DIMS = [(32, 16), (32, 64), (64, 48), (64, 64), (64, 128), (128, 32), (128, 80), (128, 128)]
GATE_SETS = [("g",), ("gk",), ("gv",), ("g", "gk"), ("g", "gv"), ("gk", "gv"), ("g", "gk", "gv")]
CASES = 40
GATED_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lattn.load_library()


def draw(i: int, bwd: bool = False) -> inputs.Workload:
    rng = np.random.default_rng(1000 + i)
    dtype = "f32" if i % 4 == 3 else "bf16"
    dims = (BWD_DIMS if bwd else DIMS)[dtype]
    dk, dv = dims[rng.integers(len(dims))]
    hkv = int(rng.choice([1, 2, 3]))
    heads = hkv * int(rng.choice([1, 2, 4]))
    num_layers = int(rng.choice([4, 12, 24]))
    layer = int(rng.integers(num_layers))
    init_std = float(rng.choice([0.0, 0.3])) or None
    reverse = bool(rng.random() < 0.5)
    if rng.random() < 0.4:  # packed, with empty and one-token sequences among them
        lens = [int(x) for x in rng.integers(0, 300, int(rng.integers(1, 7)))]
        lens[int(rng.integers(len(lens)))] = int(rng.choice([0, 1, 64, 65]))
        return inputs.Workload(f"sweep{i}", 1, sum(lens), heads, hkv, dk, dv, dtype, layer, num_layers,
                               reverse=reverse, seq_lens=lens, init_std=init_std, seed=2000 + i)
    batch = int(rng.integers(1, 4))
    seqlen = int(rng.integers(1, 400))
    return inputs.Workload(f"sweep{i}", batch, seqlen, heads, hkv, dk, dv, dtype, layer, num_layers,
                           reverse=reverse, init_std=init_std, seed=2000 + i)


@pytest.mark.parametrize("i", range(CASES))
def test_sweep_forward(i):
    w = draw(i)
    print(f"[sweep] {w}", flush=True)
    data = w.make()
    o, fs = gpu_run(w, data)
    o_ref, fs_ref = oracle_run(w, data)
    check_fwd(o.cpu().numpy(), fs.cpu().numpy(), o_ref, fs_ref, TOL[w.dtype], w.name, cu=data["cu_seqlens"])


@pytest.mark.parametrize("i", range(0, CASES, 3))
def test_sweep_backward(i):
    w = draw(i, bwd=True)
    print(f"[sweep] {w}", flush=True)
    data, grads = w.make(), w.make_grads()
    got = gpu_run_bwd(w, data, grads)
    ref = oracle_run_bwd(w, data, grads)
    for name, kind, a, b in zip(("dq", "dk", "dv", "d_initial_state"), ("tokens", "tokens", "tokens", "states"),
                                got, ref):
        check(a.cpu().numpy(), b, TOL[w.dtype], f"{w.name} {name}", kind, data["cu_seqlens"])


def draw_gated(i: int):
    rng = np.random.default_rng(5000 + i)
    dtype = "f32" if i % 4 == 3 else "bf16"
    dk, dv = GATED_DIMS[rng.integers(len(GATED_DIMS))]
    hkv = int(rng.choice([1, 2]))
    heads = hkv * int(rng.choice([1, 2, 3]))
    num_layers = 12
    layer = int(rng.integers(num_layers))
    init_std = float(rng.choice([0.0, 0.3])) or None
    reverse = bool(rng.random() < 0.5)
    gates = GATE_SETS[rng.integers(len(GATE_SETS))]
    gmax = float(rng.choice([0.1, 0.5, 3.0]))  # 3.0: summed chunk decays past the fast path's span
    use_gg = bool(rng.random() < 0.5)
    if rng.random() < 0.4:
        lens = [int(x) for x in rng.integers(0, 200, int(rng.integers(1, 6)))]
        lens[int(rng.integers(len(lens)))] = int(rng.choice([0, 1, 16, 17]))
        w = inputs.Workload(f"gsweep{i}", 1, sum(lens), heads, hkv, dk, dv, dtype, layer, num_layers,
                            reverse=reverse, seq_lens=lens, init_std=init_std, seed=6000 + i)
    else:
        w = inputs.Workload(f"gsweep{i}", int(rng.integers(1, 3)), int(rng.integers(1, 260)), heads, hkv, dk, dv,
                            dtype, layer, num_layers, reverse=reverse, init_std=init_std, seed=6000 + i)
    return w, gates, gmax, use_gg


@pytest.mark.parametrize("i", range(GATED_CASES))
def test_sweep_gated(i):
    w, which, gmax, use_gg = draw_gated(i)
    print(f"[sweep] {w} gates {which} gmax {gmax} g_gamma {use_gg}", flush=True)
    data = w.make()
    gates = w.make_gates(which, gmax)
    o, fs = gpu_run_gated(w, data, gates, use_gg)
    o_ref, fs_ref = oracle_run_gated(w, data, gates, use_gg)
    check_fwd(o.cpu().numpy(), fs.cpu().numpy(), o_ref, fs_ref, TOL[w.dtype], f"{w.name} gated", cu=data["cu_seqlens"])

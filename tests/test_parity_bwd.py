"""GPU parity of the backward pass: the HIP gradients against the fp64 oracle.

Each case compares dq, dk, dv and d_initial_state element by element with the
stated tolerance (max |gpu - oracle| <= tol * RMS(oracle)): 1e-4 for fp32 inputs,
2e-2 for bf16 inputs, over each whole tensor and over each (sequence, head) slice of
it against the slice's own RMS.  Sizes span several 64-token chunks and a ragged tail;
the full-size long-sequence case compares every gradient, with the oracle run one
batch row at a time.
"""
import numpy as np
import pytest

from decayed_recurrent_attention_amd import inputs, lattn
from tests.parity_util import TOL, Accum, check, gpu_run_bwd, oracle_run_bwd

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "d_initial_state")
KINDS = ("tokens", "tokens", "tokens", "states")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lattn.load_library()


def _compare(w, data=None, grads=None, reverse=None, g_gamma=None, tag=""):
    data = w.make() if data is None else data
    grads = w.make_grads() if grads is None else grads
    g_dev = None
    if g_gamma is not None:
        import torch

        g_dev = torch.from_numpy(g_gamma).cuda()
    got = gpu_run_bwd(w, data, grads, reverse, g_gamma=g_dev)
    ref = oracle_run_bwd(w, data, grads, reverse, g_gamma=g_gamma)
    tol = TOL[w.dtype]
    for name, kind, a, b in zip(NAMES, KINDS, got, ref):
        check(a.cpu().numpy(), b, tol, f"{w.name}{tag} {name}", kind, data["cu_seqlens"])


def test_bwd_tiny_fp32_both_directions():
    w = inputs.tiny_fp32(seqlen=200)
    w.init_std = 0.5
    data = w.make()
    _compare(w, data)
    _compare(w, data, reverse=True, tag=" rev")


def test_bwd_bf16_d64():
    w = inputs.bf16_d64(seqlen=1000)
    w.init_std = 0.3
    _compare(w)


@pytest.mark.parametrize("n", [512, 1000])
def test_bwd_long_d128(n):
    w = inputs.long_d128(seqlen=n)
    _compare(w)


@pytest.mark.parametrize("dk", [64, 128])
def test_bwd_dk_split(dk, knobs):
    """Four column blocks force the eight-wave sweeps (the dq sweep and the paired dk and
    dv sweeps) on a small problem, both directions, with an initial state."""
    knobs(lattn.LATTN_KNOB_WAVES, 4)
    w = inputs.Workload(f"bwd_dksplit{dk}", 2, 300, 4, 4, dk, dk, "bf16", 2, 12, init_std=0.4,
                        seed=32)
    data = w.make()
    _compare(w, data, tag=" nw=4")
    _compare(w, data, reverse=True, tag=" nw=4 rev")


def test_bwd_dk_split_ragged_packed(knobs):
    """The eight-wave sweeps on packed sequences with empty ones and partial chunks."""
    knobs(lattn.LATTN_KNOB_WAVES, 4)
    lens = [0, 1, 63, 64, 65, 130, 0, 7]
    w = inputs.Workload("bwd_dksplit_ragged", 1, sum(lens), 4, 4, 128, 64, "bf16", 3, 12,
                        seq_lens=lens, init_std=0.3, seed=34)
    _compare(w, tag=" nw=4")
    _compare(w, reverse=True, tag=" nw=4 rev")


def test_bwd_d192():
    w = inputs.d192(seqlen=700)
    _compare(w)


@pytest.mark.parametrize("reverse", [False, True])
def test_bwd_varlen_gqa(reverse):
    w = inputs.varlen_gqa(reverse=reverse, num_seqs=6, lo=1, hi=700, seed=21)
    _compare(w)


def test_bwd_ragged_packed_with_empty_sequences():
    lens = [0, 1, 63, 64, 65, 130, 0, 7]
    w = inputs.Workload("bwd_ragged", 1, sum(lens), 8, 2, 64, 64, "bf16", 3, 12, seq_lens=lens,
                        init_std=0.3, seed=22)
    _compare(w)
    _compare(w, reverse=True, tag=" rev")


@pytest.mark.parametrize("dk,dv,dtype", [(64, 128, "bf16"), (128, 64, "bf16"), (32, 64, "f32"),
                                         (64, 32, "f32")])
def test_bwd_unequal_head_dims(dk, dv, dtype):
    w = inputs.Workload(f"bwd_dk{dk}_dv{dv}_{dtype}", 2, 300, 4, 2, dk, dv, dtype, 4, 12,
                        init_std=0.2, seed=23)
    _compare(w)


def test_bwd_strong_decay_and_no_decay():
    w = inputs.Workload("bwd_decay", 1, 700, 4, 4, 64, 64, "bf16", 0, 1, init_std=1.0, seed=24)
    g = np.array([-0.0, -3.0, -30.0, -200.0], dtype=np.float32)
    _compare(w, g_gamma=g)


def test_bwd_without_state_gradients():
    """No initial state, no final-state gradient, d_initial_state not requested."""
    w = inputs.Workload("bwd_plain", 2, 333, 4, 4, 128, 128, "bf16", 2, 12, seed=25)
    data = w.make()
    grads = w.make_grads(final_std=None)
    dq, dk, dv, d_init = gpu_run_bwd(w, data, grads, want_d_init=False)
    assert d_init is None
    ref = oracle_run_bwd(w, data, grads)
    for name, a, b in zip(NAMES[:3], (dq, dk, dv), ref[:3]):
        check(a.cpu().numpy(), b, TOL["bf16"], f"bwd_plain {name}", "tokens")


def test_bwd_long_d128_n32768_whole():
    """Full-size long sequence (B=4, H=32, d=128, N=32768), every gradient compared with the
    oracle, which runs one batch row at a time to bound host memory."""
    import oracle

    w = inputs.long_d128(seqlen=32768)
    data = w.make()
    grads = w.make_grads()
    got = gpu_run_bwd(w, data, grads)
    orc = oracle.load()
    g = orc.lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers)
    accs = [Accum(f"n32768 {name}") for name in NAMES]
    for b in range(w.batch):
        row = lambda a: np.ascontiguousarray(a[b:b + 1])
        ref = orc.recurrent_bwd(row(data["q"]), row(data["k"]), row(data["v"]), g, w.scale, row(grads["d_o"]),
                                row(grads["d_final_state"]))
        for acc, kind, x, y in zip(accs, KINDS, got, ref):
            if kind == "tokens":
                acc.add_tokens(x[b:b + 1].cpu().numpy(), y, row0=b)
            else:
                acc.add_states(x[b:b + 1].cpu().numpy(), y, n0=b)
        del ref
    for acc in accs:
        acc.finish(TOL["bf16"])


def test_bwd_deterministic():
    import torch

    w = inputs.varlen_gqa(num_seqs=5, lo=60, hi=700, seed=26)
    data, grads = w.make(), w.make_grads()
    a = gpu_run_bwd(w, data, grads)
    b = gpu_run_bwd(w, data, grads)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("reverse", [False, True])
def test_bwd_paired_sweeps_equal_separate(reverse, knobs):
    """bf16 with dk = dv and no grouped heads runs the dk and dv sweeps as one launch;
    every workgroup does the same arithmetic either way, so the gradients are
    bit-identical to two launches (knob LATTN_KNOB_BWD_PAIR = 0), and both meet the oracle."""
    import torch

    w = inputs.Workload("bwd_pair", 2, 700, 4, 4, 64, 64, "bf16", 2, 12, reverse=reverse, init_std=0.3, seed=27)
    data, grads = w.make(), w.make_grads()
    a = gpu_run_bwd(w, data, grads)
    knobs(lattn.LATTN_KNOB_BWD_PAIR, 0)
    b = gpu_run_bwd(w, data, grads)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    ref = oracle_run_bwd(w, data, grads)
    for got, exp, name, kind in zip(a, ref, NAMES, KINDS):
        check(got.cpu().numpy(), exp, TOL["bf16"], f"bwd_pair{' rev' if reverse else ''} {name}", kind)

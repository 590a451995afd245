"""GPU parity: the HIP path against the fp64 oracle, element by element.

Runs on an MI355X through the C ABI (via the Python binding).  Sizes are chosen so
that the oracle finishes in seconds while spanning several 64-token chunks and a
ragged tail.  The long-sequence workload is compared whole at every N of its sweep,
N = 32768 included, in the launch configuration that the benchmark times (the oracle
runs one batch row at a time there).  Every comparison applies the bar to the whole
tensor and to every (sequence, head) slice against its own RMS.
"""
import os

import numpy as np
import pytest

from decayed_recurrent_attention_amd import inputs, lattn
from tests.parity_util import TOL, Accum, check, check_fwd, gpu_run, oracle_run, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lattn.load_library()


def _compare(w, data, reverse=None, tag=""):
    o, fs = gpu_run(w, data, reverse)
    o_ref, fs_ref = oracle_run(w, data, reverse)
    check_fwd(o.cpu().numpy(), fs.cpu().numpy(), o_ref, fs_ref, TOL[w.dtype], w.name + tag,
              cu=data["cu_seqlens"])


# -- the five workloads ------------------------------------------------------------
def test_tiny_fp32():
    w = inputs.tiny_fp32()
    _compare(w, w.make())


def test_tiny_fp32_reverse_with_state():
    w = inputs.tiny_fp32(seqlen=200)
    w.init_std = 0.5
    _compare(w, w.make(), reverse=True, tag=" rev+init")


def test_bf16_d64():
    w = inputs.bf16_d64()
    _compare(w, w.make())


@pytest.mark.parametrize("n", [512, 1024, 2048, 4096])
def test_long_d128_full(n):
    w = inputs.long_d128(seqlen=n)
    _compare(w, w.make())


def test_d192():
    w = inputs.d192()
    _compare(w, w.make())


@pytest.mark.parametrize("reverse", [False, True])
def test_varlen_gqa(reverse):
    w = inputs.varlen_gqa(reverse=reverse)
    _compare(w, w.make())


@pytest.mark.parametrize("n", [8192, 16384, 32768])
def test_long_d128_whole_tensor_rowwise(n):
    """The long-sequence workload (B=4, H=32, d=128) at N = 8192, 16384 and 32768, run as
    the benchmark runs it (one call over the whole batch); every output is compared with
    the oracle, which runs one batch row at a time to bound host memory."""
    import torch

    w = inputs.long_d128(seqlen=n)
    data = w.make()
    o, fs = gpu_run(w, data)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(fs).all().item()
    orc = __import__("oracle").load()
    g = orc.lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers)
    acc_o, acc_s = Accum(f"{w.name} o"), Accum(f"{w.name} final_state")
    for b in range(w.batch):
        row = lambda a: np.ascontiguousarray(a[b:b + 1])
        o_ref, fs_ref = orc.recurrent_fwd(row(data["q"]), row(data["k"]), row(data["v"]), g, w.scale)
        acc_o.add_tokens(o[b:b + 1].cpu().numpy(), o_ref, row0=b)
        acc_s.add_states(fs[b:b + 1].cpu().numpy(), fs_ref, n0=b)
        del o_ref, fs_ref
    acc_o.finish(TOL["bf16"])
    acc_s.finish(TOL["bf16"])


# -- edge cases ----------------------------------------------------------------------
@pytest.mark.parametrize("reverse", [False, True])
def test_ragged_packed_lengths(reverse):
    lens = [0, 1, 63, 64, 65, 127, 200, 2, 0, 129]
    w = inputs.Workload("ragged_packed", 1, sum(lens), 8, 2, 64, 64, "bf16", 3, 12,
                        reverse=reverse, seq_lens=lens, init_std=0.3, seed=3)
    _compare(w, w.make(), tag=" rev" if reverse else "")


def test_ragged_fixed_length_reverse_with_state():
    w = inputs.Workload("ragged_fixed", 2, 1000, 4, 4, 128, 128, "bf16", 2, 12, reverse=True,
                        init_std=1.0, seed=4)
    _compare(w, w.make())


@pytest.mark.parametrize("dk,dv,dtype", [(64, 128, "bf16"), (128, 64, "bf16"), (32, 16, "bf16"),
                                         (256, 64, "bf16"), (64, 32, "f32"), (128, 64, "f32"),
                                         (32, 48, "f32")])
def test_unequal_head_dims(dk, dv, dtype):
    w = inputs.Workload(f"dk{dk}_dv{dv}_{dtype}", 2, 300, 4, 2, dk, dv, dtype, 4, 12,
                        init_std=0.2, seed=5)
    _compare(w, w.make())


@pytest.mark.parametrize("dk,dv,dtype", [(256, 256, "bf16"), (192, 256, "bf16"), (128, 256, "f32")])
def test_largest_head_dims(dk, dv, dtype):
    """The largest supported head dims per dtype (dv up to 256), both directions of the
    work, GQA, ragged length."""
    w = inputs.Workload(f"max_dk{dk}_dv{dv}_{dtype}", 2, 333, 4, 2, dk, dv, dtype, 3, 12,
                        init_std=0.2, seed=8)
    _compare(w, w.make())


@pytest.mark.parametrize("nw", ["1", "2", "4"])
def test_workgroup_widths(nw, knobs):
    knobs(lattn.LATTN_KNOB_WAVES, int(nw))
    w = inputs.Workload(f"nw{nw}", 2, 333, 4, 4, 64, 64, "bf16", 1, 12, init_std=0.1, seed=6)
    _compare(w, w.make(), tag=f" nw={nw}")


@pytest.mark.parametrize("dk,reverse", [(128, False), (128, True), (64, True)])
def test_dk_split_small(dk, reverse, knobs):
    """Four column blocks force the eight-wave kernel (two waves per column block, each
    with half of the dk rows) on a small ragged GQA problem with an initial state."""
    knobs(lattn.LATTN_KNOB_WAVES, 4)
    w = inputs.Workload(f"dksplit{dk}", 2, 333, 4, 2, dk, 64, "bf16", 2, 12, reverse=reverse,
                        init_std=0.5, seed=31)
    _compare(w, w.make(), tag=" nw=4")


@pytest.mark.parametrize("reverse", [False, True])
def test_dk_split_ragged_packed(reverse, knobs):
    """The eight-wave kernel on packed sequences of 0, 1, 63, 64, 65, ... tokens (empty
    sequences, single tokens, partial chunks) with GQA and an initial state."""
    knobs(lattn.LATTN_KNOB_WAVES, 4)
    lens = [0, 1, 63, 64, 65, 127, 200, 2, 0, 129]
    w = inputs.Workload("dksplit_ragged", 1, sum(lens), 8, 2, 128, 64, "bf16", 3, 12,
                        reverse=reverse, seq_lens=lens, init_std=0.3, seed=33)
    _compare(w, w.make(), tag=" nw=4" + (" rev" if reverse else ""))


def test_no_decay_long():
    """Last layer: g = 0 for every head, the state only grows."""
    w = inputs.Workload("no_decay", 1, 8192, 4, 4, 128, 128, "bf16", 12, 12, seed=7)
    _compare(w, w.make())


def test_explicit_g_gamma_strong_decay():
    import torch

    w = inputs.Workload("strong_decay", 1, 700, 4, 4, 64, 64, "bf16", 0, 1, init_std=1.0, seed=8)
    data = w.make()
    g = np.array([-0.0, -3.0, -30.0, -200.0], dtype=np.float32)
    o, fs = gpu_run(w, data, g_gamma=torch.from_numpy(g).cuda())
    o_ref, fs_ref = oracle_run(w, data, g_gamma=g)
    check_fwd(o.cpu().numpy(), fs.cpu().numpy(), o_ref, fs_ref, TOL["bf16"], "strong decay")


def test_empty_sequence_batch():
    import torch

    w = inputs.Workload("empty", 2, 0, 4, 4, 64, 64, "bf16", 1, 12, init_std=1.0, seed=9)
    data = w.make()
    o, fs = gpu_run(w, data)
    assert o.shape == (2, 0, 4, 64)
    assert torch.equal(fs.cpu(), torch.from_numpy(data["initial_state"]))


def test_chained_segments_match_whole():
    """Splitting a sequence and chaining final_state -> initial_state matches one call."""
    import torch

    w = inputs.Workload("chain", 2, 1100, 4, 4, 128, 128, "bf16", 5, 12, seed=10)
    data = w.make()
    q, k, v = (to_device(data[n], "bf16") for n in ("q", "k", "v"))
    o, fs = lattn.lightning_attn(q, k, v, 5, 12)
    m = 517
    o1, fs1 = lattn.lightning_attn(q[:, :m], k[:, :m], v[:, :m], 5, 12)
    o2, fs2 = lattn.lightning_attn(q[:, m:], k[:, m:], v[:, m:], 5, 12, initial_state=fs1)
    o_ref, fs_ref = oracle_run(w, data)
    check_fwd(torch.cat([o1, o2], 1).cpu().numpy(), fs2.cpu().numpy(), o_ref, fs_ref, TOL["bf16"],
              "chained")
    assert (o - torch.cat([o1, o2], 1)).abs().max().item() <= 1e-3 * o.abs().max().item()


def test_deterministic():
    import torch

    w = inputs.varlen_gqa(num_seqs=5, lo=60, hi=700, seed=11)
    data = w.make()
    o1, fs1 = gpu_run(w, data)
    o2, fs2 = gpu_run(w, data)
    assert torch.equal(o1, o2) and torch.equal(fs1, fs2)


def test_varlen_3d_input_matches_4d():
    import torch

    w = inputs.varlen_gqa(num_seqs=4, lo=10, hi=300, seed=12)
    data = w.make()
    o4, fs4 = gpu_run(w, data)
    q, k, v = (to_device(data[n], "bf16")[0] for n in ("q", "k", "v"))
    o3, fs3 = lattn.lightning_attn(q, k, v, w.layer_idx, w.num_layers, softmax_scale=w.scale,
                                   initial_state=to_device(data["initial_state"], "f32"),
                                   cu_seqlens=data["cu_seqlens"])
    assert torch.equal(o3, o4[0]) and torch.equal(fs3, fs4)


# -- intra-sequence split (fixed-length bf16 input with few (row, head) pairs) -------------
@pytest.mark.parametrize("reverse", [False, True])
def test_split_forced_segments(reverse, knobs):
    knobs(lattn.LATTN_KNOB_SPLIT, 3)  # 16 chunks -> 3 segments of 6, 6 and 4 chunks
    w = inputs.Workload("split3", 2, 1000, 4, 4, 64, 64, "bf16", 3, 12, reverse=reverse,
                        init_std=0.5, seed=41)
    _compare(w, w.make(), tag=" rev" if reverse else "")


@pytest.mark.parametrize("segments", [16, 17])
@pytest.mark.parametrize("reverse", [False, True])
def test_split_chain_in_main_pass_or_scan(segments, reverse, knobs):
    """Sixteen one-chunk segments: the main pass chains up to fifteen slots itself;
    seventeen: the scan chains them first.  Both against the oracle, in both directions."""
    knobs(lattn.LATTN_KNOB_SPLIT, segments)
    w = inputs.Workload(f"split{segments}_d64", 1, 64 * segments, 2, 2, 64, 64, "bf16", 3, 24, reverse=reverse,
                        init_std=0.3, seed=45 + segments)
    _compare(w, w.make(), tag=" rev" if reverse else "")


@pytest.mark.parametrize("dk,dv", [(256, 256), (192, 256)])
@pytest.mark.parametrize("reverse", [False, True])
def test_split_widest_heads(dk, dv, reverse, knobs):
    """The state-only pass with three K/V stages and one workgroup per compute unit (dk 192
    and 256), with GQA and an initial state."""
    knobs(lattn.LATTN_KNOB_SPLIT, 3)
    w = inputs.Workload(f"split3_dk{dk}_dv{dv}", 1, 1400, 4, 2, dk, dv, "bf16", 5, 12, reverse=reverse,
                        init_std=0.2, seed=47)
    _compare(w, w.make(), tag=" rev" if reverse else "")


def test_split_forced_gqa_unequal_dims(knobs):
    knobs(lattn.LATTN_KNOB_SPLIT, 5)
    w = inputs.Workload("split5_gqa", 1, 777, 8, 2, 128, 64, "bf16", 6, 12, init_std=0.3, seed=43)
    _compare(w, w.make())


@pytest.mark.parametrize("reverse", [False, True])
def test_split_automatic_long_sequence(reverse, knobs):
    w = inputs.Workload("split_auto", 1, 16384, 4, 4, 128, 128, "bf16", 1, 12, reverse=reverse,
                        init_std=0.2, seed=42)
    prob = lattn.LattnProblem(1, 16384, 4, 4, 128, 128, 0, lattn.LATTN_BF16, lattn.LATTN_F32)
    assert lattn.lattn_fwd_workspace_size(prob) > 0, "expected the split path"
    _compare(w, w.make(), tag=" rev" if reverse else "")


def test_split_matches_unsplit(knobs):
    """Split and unsplit runs agree to rounding (different summation order)."""
    w = inputs.Workload("split_vs", 2, 3000, 2, 2, 128, 128, "bf16", 2, 12, init_std=0.5, seed=44)
    data = w.make()
    knobs(lattn.LATTN_KNOB_SPLIT, 0)
    o0, f0 = gpu_run(w, data)
    knobs(lattn.LATTN_KNOB_SPLIT, 4)
    o1, f1 = gpu_run(w, data)
    scale_o = float(o0.abs().max())
    assert float((o0 - o1).abs().max()) <= 1e-4 * scale_o
    assert float((f0 - f1).abs().max()) <= 1e-4 * float(f0.abs().max())


def test_library_is_the_one_loaded():
    """The HIP library in the package directory is what runs (no fallback)."""
    lib = lattn.load_library()
    assert os.path.samefile(lib._name, lattn.LIB_PATH)


# -- packed input split along its sequences (device-planned segments) -----------------------
@pytest.mark.parametrize("reverse", [False, True])
def test_packed_split_forced(reverse, knobs):
    """Every sequence of at least two chunks cut into up to 3 segments: empty, short and
    ragged sequences, GQA, dk != dv, an initial state, both directions."""
    knobs(lattn.LATTN_KNOB_SPLIT, 3)
    lens = [0, 1, 63, 64, 65, 127, 200, 2, 0, 129, 700, 1000]
    w = inputs.Workload("packed_split3", 1, sum(lens), 8, 2, 128, 64, "bf16", 3, 12, reverse=reverse,
                        seq_lens=lens, init_std=0.3, seed=81)
    _compare(w, w.make(), tag=" rev" if reverse else "")


@pytest.mark.parametrize("reverse", [False, True])
def test_packed_split_skewed_automatic(reverse):
    """One long sequence among short ones: the planner cuts the long one (its chunks exceed
    the balanced load per compute unit) and leaves the rest whole."""
    lens = [9000, 70, 130, 64, 1, 300, 0, 250, 90, 128]
    w = inputs.Workload("packed_skewed", 1, sum(lens), 4, 2, 128, 128, "bf16", 2, 12, reverse=reverse,
                        seq_lens=lens, init_std=0.2, seed=82)
    prob = lattn.LattnProblem(1, w.seqlen, 4, 2, 128, 128, len(lens), lattn.LATTN_BF16, lattn.LATTN_F32)
    assert lattn.lattn_fwd_workspace_size(prob) > 4096, "expected the planner's workspace"
    _compare(w, w.make(), tag=" rev" if reverse else "")


def test_packed_split_matches_unsplit(knobs):
    """The split and unsplit packed runs agree to rounding (different summation order)."""
    lens = [5000, 40, 700, 3, 1200]
    w = inputs.Workload("packed_split_vs", 1, sum(lens), 4, 4, 64, 64, "bf16", 5, 12, seq_lens=lens,
                        init_std=0.5, seed=83)
    data = w.make()
    knobs(lattn.LATTN_KNOB_SPLIT, 0)
    o0, f0 = gpu_run(w, data)
    knobs(lattn.LATTN_KNOB_SPLIT, lattn.LATTN_KNOB_AUTO)
    o1, f1 = gpu_run(w, data)
    knobs(lattn.LATTN_KNOB_SPLIT, 6)
    o2, f2 = gpu_run(w, data)
    for o, f in ((o1, f1), (o2, f2)):
        assert float((o0 - o).abs().max()) <= 1e-4 * float(o0.abs().max())
        assert float((f0 - f).abs().max()) <= 1e-4 * float(f0.abs().max())

"""GPU checks of the bf16 output mode of lattn_fwd (bf16 input, o in bf16).

Each element of the bf16 o must be the round-to-nearest-even of the float32 result that
the same call with a float32 o returns (compared bit for bit), and the final state must
be bit-identical.  Against the fp64 oracle the bf16 o is bounded by the float32 bar plus
the rounding itself: |o - o_ref| <= 2e-2 * RMS + 2^-8 * |o_ref| per element (a bf16
rounding moves a value by at most 2^-8 of itself), with RMS that of the whole tensor and,
separately, that of the element's own (sequence, head) slice.
"""
import numpy as np
import pytest

from decayed_recurrent_attention_amd import inputs, lattn
from tests.parity_util import TOL, check, oracle_run, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lattn.load_library()


def _both(w, data, reverse):
    import torch

    q, k, v = (to_device(data[n], w.dtype) for n in ("q", "k", "v"))
    init = to_device(data["initial_state"], "f32")
    kw = dict(softmax_scale=w.scale, initial_state=init, reverse=reverse, cu_seqlens=data["cu_seqlens"])
    o32, fs32 = lattn.lightning_attn(q, k, v, w.layer_idx, w.num_layers, **kw)
    o16, fs16 = lattn.lightning_attn(q, k, v, w.layer_idx, w.num_layers, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    return o32, fs32, o16, fs16


def _check(w, data, reverse, tag):
    import torch

    o32, fs32, o16, fs16 = _both(w, data, reverse)
    assert o16.dtype == torch.bfloat16 and o16.shape == o32.shape
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16)), f"{tag}: o is not RNE(f32 o)"
    assert torch.equal(fs16, fs32), f"{tag}: final_state differs"
    o_ref, fs_ref = oracle_run(w, data, reverse=reverse)
    got = o16.float().cpu().numpy().astype(np.float64)
    ref = np.asarray(o_ref, dtype=np.float64)

    def bound(g, r, what):
        if r.size:
            rms = float(np.sqrt(np.mean(r * r)))
            excess = np.abs(g - r) - (TOL["bf16"] * rms + 2.0 ** -8 * np.abs(r))
            assert excess.max() <= 0.0, f"{tag}: bf16 o ({what}) exceeds the bound by {excess.max():.3e}"

    bound(got, ref, "whole tensor")
    cu = data["cu_seqlens"]
    rows = [(b, 0, ref.shape[1]) for b in range(ref.shape[0])] if cu is None else \
        [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    for b, t0, t1 in rows:
        for h in range(ref.shape[2]):
            bound(got[b, t0:t1, h], ref[b, t0:t1, h], f"row {b} tokens {t0}:{t1} head {h}")
    check(fs16.cpu().numpy(), fs_ref, TOL["bf16"], f"{tag} final_state", "states")


@pytest.mark.parametrize("reverse", [False, True])
def test_bf16_out_dk_split_gqa_ragged(reverse, knobs):
    knobs(lattn.LATTN_KNOB_WAVES, 4)  # the eight-wave kernel
    w = inputs.Workload("bf16out_split", 2, 333, 4, 2, 128, 64, "bf16", 2, 12, reverse=reverse,
                        init_std=0.5, seed=41)
    _check(w, w.make(), reverse, w.name)


@pytest.mark.parametrize("reverse", [False, True])
def test_bf16_out_packed(reverse):
    lens = [0, 1, 63, 64, 65, 127, 200, 2, 0, 129]
    w = inputs.Workload("bf16out_packed", 1, sum(lens), 8, 2, 64, 64, "bf16", 3, 12, reverse=reverse,
                        seq_lens=lens, init_std=0.3, seed=42)
    _check(w, w.make(), reverse, w.name)


def test_bf16_out_intra_sequence_split(knobs):
    knobs(lattn.LATTN_KNOB_SPLIT, 3)
    w = inputs.Workload("bf16out_seqsplit", 2, 1000, 4, 4, 64, 64, "bf16", 1, 12, init_std=0.2, seed=43)
    _check(w, w.make(), False, w.name)


def test_bf16_out_long_d128():
    """The benchmark's head shape (B4 H32 d128, layer 0 of 12) at N = 512."""
    w = inputs.long_d128(seqlen=512)
    _check(w, w.make(), False, w.name)


def test_bf16_out_rejected_where_unsupported():
    import torch

    w = inputs.Workload("bf16out_f32", 1, 64, 2, 2, 32, 32, "f32", 1, 12, seed=44)
    data = w.make()
    q, k, v = (to_device(data[n], w.dtype) for n in ("q", "k", "v"))
    with pytest.raises(ValueError):
        lattn.lightning_attn(q, k, v, 1, 12, out_dtype=torch.bfloat16)
    g = torch.zeros_like(q)
    with pytest.raises(ValueError):
        lattn.recurrent(q.bfloat16(), k.bfloat16(), v.bfloat16(), g=g.bfloat16(), out_dtype=torch.bfloat16)

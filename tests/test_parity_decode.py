"""GPU parity of the decoding step (lattn_decode) against the fp64 oracle.

A decoding step is the recurrence advanced by one token, so its oracle is the
forward oracle at seqlen 1 with the incoming state as initial_state.  Tolerance as
for the forward: max |gpu - oracle| <= tol * RMS(oracle) (1e-4 fp32 inputs, 2e-2 bf16
inputs), over each whole tensor and over each (sequence, head) slice.
"""
import numpy as np
import pytest

from decayed_recurrent_attention_amd import inputs, lattn
from tests.parity_util import TOL, check, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lattn.load_library()


def _g(w):
    return lattn.lattn_lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers)


def _one_step(w, g=None, with_state=True):
    import torch
    import oracle

    data = w.make()
    g = _g(w) if g is None else g
    q, k, v = (to_device(data[n], w.dtype)[:, 0] for n in ("q", "k", "v"))
    state = to_device(data["initial_state"], "f32") if with_state else None
    o, s_new = lattn.decode_step(q, k, v, state, g_gamma=torch.from_numpy(g).cuda(),
                                 softmax_scale=w.scale, in_place=False)
    o_ref, s_ref = oracle.load().recurrent_fwd(data["q"], data["k"], data["v"], g, w.scale,
                                               initial_state=data["initial_state"] if with_state else None)
    tol = TOL[w.dtype]
    check(o.cpu().numpy(), o_ref[:, 0], tol, f"{w.name} decode o", "rows")
    check(s_new.cpu().numpy(), s_ref, tol, f"{w.name} decode state", "states")


@pytest.mark.parametrize("B,H,Hkv,dk,dv,dtype", [
    (8, 8, 2, 64, 64, "bf16"),
    (4, 32, 32, 128, 128, "bf16"),
    (3, 4, 4, 256, 256, "bf16"),
    (5, 6, 3, 128, 48, "bf16"),   # 16-column value blocks
    (2, 4, 1, 32, 96, "f32"),     # 32-column value blocks
    (7, 2, 2, 16, 16, "f32"),
])
def test_decode_one_step(B, H, Hkv, dk, dv, dtype):
    w = inputs.Workload(f"dec_b{B}_h{H}_{dk}x{dv}_{dtype}", B, 1, H, Hkv, dk, dv, dtype, 4, 12,
                        init_std=0.5, seed=31)
    _one_step(w)


def test_decode_zero_state_and_decay_extremes():
    w = inputs.Workload("dec_zero", 6, 1, 4, 4, 64, 64, "bf16", 0, 1, init_std=1.0, seed=32)
    _one_step(w, with_state=False)
    _one_step(w, g=np.array([-0.0, -3.0, -30.0, -200.0], dtype=np.float32))


def test_decode_bench_shape():
    """The decode batch the benchmark times: 128 sequences, H=32, d=128, bf16."""
    w = inputs.Workload("dec_bench", 128, 1, 32, 32, 128, 128, "bf16", 0, 12, init_std=0.5, seed=33)
    _one_step(w)


def test_decode_in_place_matches_out_of_place():
    import torch

    w = inputs.Workload("dec_inplace", 4, 1, 8, 8, 128, 128, "bf16", 2, 12, init_std=0.5, seed=34)
    data = w.make()
    q, k, v = (to_device(data[n], w.dtype)[:, 0] for n in ("q", "k", "v"))
    g = torch.from_numpy(_g(w)).cuda()
    s0 = to_device(data["initial_state"], "f32")
    o1, s1 = lattn.decode_step(q, k, v, s0.clone(), g_gamma=g, softmax_scale=w.scale, in_place=False)
    s_in = s0.clone()
    o2, s2 = lattn.decode_step(q, k, v, s_in, g_gamma=g, softmax_scale=w.scale, in_place=True)
    assert s2.data_ptr() == s_in.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps_match_the_sequence(dtype):
    """150 decoding steps from an initial state equal the recurrence over 150 tokens."""
    import torch
    import oracle

    T = 150
    w = inputs.Workload(f"dec_seq_{dtype}", 3, T, 4, 2, 64, 64, dtype, 5, 12, init_std=0.3, seed=35)
    data = w.make()
    g = _g(w)
    q, k, v = (to_device(data[n], w.dtype) for n in ("q", "k", "v"))
    state = to_device(data["initial_state"], "f32")
    gd = torch.from_numpy(g).cuda()
    outs = []
    for t in range(T):
        o, state = lattn.decode_step(q[:, t], k[:, t], v[:, t], state, g_gamma=gd, softmax_scale=w.scale)
        outs.append(o)
    o_all = torch.stack(outs, 1)
    o_ref, s_ref = oracle.load().recurrent_fwd(data["q"], data["k"], data["v"], g, w.scale,
                                               initial_state=data["initial_state"])
    tol = TOL[dtype]
    check(o_all.cpu().numpy(), o_ref, tol, f"{w.name} o over {T} steps", "tokens")
    check(state.cpu().numpy(), s_ref, tol, f"{w.name} state after {T} steps", "states")

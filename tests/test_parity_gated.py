"""GPU parity of the gated recurrence (lattn_fwd_gated: g, gk, gv log-decay gates)
against the fp64 oracle.  Tolerance as for the forward: max |gpu - oracle| <= tol *
RMS(oracle), 1e-4 for fp32 inputs and 2e-2 for bf16 inputs, over each whole tensor and
over each (sequence, head) slice against its own RMS (the bf16 cases sit far inside
their bar)."""
import numpy as np
import pytest

from decayed_recurrent_attention_amd import inputs, lattn
from tests.parity_util import TOL, Accum, check, check_fwd, gpu_run_gated, oracle_run_gated, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lattn.load_library()


def _run(w, data, gates, use_gg=True, reverse=None):
    o, fs = gpu_run_gated(w, data, gates, use_gg, reverse)
    o_ref, fs_ref = oracle_run_gated(w, data, gates, use_gg, reverse)
    return o, fs, o_ref, fs_ref


def _compare(w, which, gmax=0.5, use_gg=True, reverse=None, tag=""):
    data = w.make()
    gates = w.make_gates(which, gmax)
    o, fs, o_ref, fs_ref = _run(w, data, gates, use_gg, reverse)
    check_fwd(o.cpu().numpy(), fs.cpu().numpy(), o_ref, fs_ref, TOL[w.dtype], f"{w.name}{tag} gated",
              cu=data["cu_seqlens"])


@pytest.mark.parametrize("which", [("g",), ("gk", "gv"), ("g", "gk", "gv")])
@pytest.mark.parametrize("reverse", [False, True])
def test_gated_fp32(which, reverse):
    w = inputs.Workload("gated_f32", 2, 150, 4, 2, 32, 32, "f32", 5, 12, init_std=0.5, seed=51)
    _compare(w, which, reverse=reverse, tag=f" {'+'.join(which)}{' rev' if reverse else ''}")


def test_gla_bf16_d64_gqa():
    w = inputs.Workload("gla_d64", 2, 1000, 8, 4, 64, 64, "bf16", 3, 12, init_std=0.3, seed=52)
    _compare(w, ("g",), use_gg=False)


def test_gated_bf16_d128_value_gates():
    w = inputs.Workload("gated_d128", 2, 2100, 4, 4, 128, 128, "bf16", 0, 12, init_std=0.2, seed=53)
    _compare(w, ("g", "gv"), gmax=0.2)


@pytest.mark.parametrize("reverse", [False, True])
def test_gated_packed_ragged(reverse):
    lens = [0, 1, 15, 16, 17, 100, 0, 33]
    w = inputs.Workload("gated_packed", 1, sum(lens), 4, 2, 64, 48, "bf16", 2, 12, seq_lens=lens,
                        reverse=reverse, init_std=0.4, seed=54)
    _compare(w, ("g", "gk", "gv"), tag=" rev" if reverse else "")


def test_gated_narrow_value_block():
    """dv not a multiple of 64: one-wave workgroups of 16 columns."""
    w = inputs.Workload("gated_dv80", 2, 300, 2, 2, 128, 80, "bf16", 4, 12, init_std=0.3, seed=55)
    _compare(w, ("g", "gv"))


def test_gated_strong_gates():
    """Per-token decays down to e^-6: cumulative exponents reach about -96 per chunk."""
    w = inputs.Workload("gated_strong", 1, 500, 4, 4, 64, 64, "bf16", 1, 12, init_std=1.0, seed=56)
    _compare(w, ("g", "gv"), gmax=6.0)


def test_gated_constant_gate_equals_lightning():
    """gk constant per head equals g_gamma: the gated and Lightning kernels agree."""
    import torch

    w = inputs.Workload("gated_const", 2, 700, 4, 4, 64, 64, "bf16", 6, 12, init_std=0.3, seed=57)
    data = w.make()
    g = np.array([-0.0, -0.5, -1.25, -3.0], dtype=np.float32)
    gk = np.broadcast_to(g[None, None, :, None], (w.batch, w.seqlen, w.num_heads, w.dk)).astype(np.float32)
    gk_w = inputs.bf16_words(gk)  # these values are exact in bf16
    q, k, v = (to_device(data[n], "bf16") for n in ("q", "k", "v"))
    init = to_device(data["initial_state"], "f32")
    o1, f1 = lattn.recurrent_gated(q, k, v, gk=to_device(gk_w, "bf16"), softmax_scale=w.scale, initial_state=init)
    o2, f2 = lattn.recurrent(q, k, v, g_gamma=torch.from_numpy(g).cuda(), softmax_scale=w.scale,
                             initial_state=init)
    import oracle

    o_ref, f_ref = oracle.load().recurrent_fwd(data["q"], data["k"], data["v"], g, w.scale,
                                               initial_state=data["initial_state"])
    check_fwd(o1.cpu().numpy(), f1.cpu().numpy(), o_ref, f_ref, TOL["bf16"], "constant gate (gated kernel)")
    check_fwd(o2.cpu().numpy(), f2.cpu().numpy(), o_ref, f_ref, TOL["bf16"], "constant gate (Lightning kernel)")


def test_gla_long_d128_whole():
    """The benchmark's gated workload (B4 H32 d128 N32768 bf16, g gates), every output
    compared with the oracle, which runs one batch row at a time."""
    w = inputs.long_d128(seqlen=32768)
    data = w.make()
    gates = w.make_gates(("g",), 0.1)
    dev = {n: to_device(data[n], "bf16") for n in ("q", "k", "v")}
    o, fs = lattn.recurrent_gla(dev["q"], dev["k"], dev["v"], g=to_device(gates["g"], "bf16"),
                                softmax_scale=w.scale)
    import oracle

    orc = oracle.load()
    acc_o, acc_s = Accum("gla n32768 o"), Accum("gla n32768 final_state")
    for b in range(w.batch):
        row = lambda a: np.ascontiguousarray(a[b:b + 1])
        o_ref, fs_ref = orc.recurrent_gated_fwd(row(data["q"]), row(data["k"]), row(data["v"]), g=row(gates["g"]),
                                                scale=w.scale)
        acc_o.add_tokens(o[b:b + 1].cpu().numpy(), o_ref, row0=b)
        acc_s.add_states(fs[b:b + 1].cpu().numpy(), fs_ref, n0=b)
        del o_ref, fs_ref
    acc_o.finish(TOL["bf16"])
    acc_s.finish(TOL["bf16"])


def test_gated_bf16_g_plus_gk_d128_reverse():
    """g and gk both given (summed into one fp32 key gate first), fixed length, reverse,
    GQA, initial state and g_gamma."""
    w = inputs.Workload("gated_ggk", 2, 777, 4, 2, 128, 128, "bf16", 3, 12, reverse=True, init_std=0.3, seed=58)
    _compare(w, ("g", "gk"), gmax=0.3)


@pytest.mark.parametrize("shape", [(32, 64), (32, 32), (128, 256), (64, 48)])
def test_gated_bf16_head_dims(shape):
    """dk 32 / 64 / 128 with one- and four-wave value blocks (dv 32, 48, 64, 256)."""
    dk, dv = shape
    w = inputs.Workload(f"gated_dk{dk}_dv{dv}", 2, 321, 4, 4, dk, dv, "bf16", 2, 12, init_std=0.3, seed=59 + dk + dv)
    _compare(w, ("g", "gv"), gmax=0.4, tag=f" dk{dk} dv{dv}")


@pytest.mark.parametrize("T", [1, 5, 16, 17, 31, 32, 33, 48, 64])
def test_gated_bf16_short(T):
    """One to four chunks: the producers' prologue, the last-chunk repeats past the end and
    the pairing of steps for odd and even chunk counts."""
    w = inputs.Workload(f"gated_short{T}", 3, T, 4, 4, 64, 64, "bf16", 2, 12, init_std=0.5, seed=61 + T)
    _compare(w, ("g", "gv"), gmax=0.5, tag=f" T{T}")


def _banded_gates(w, strong_k, strong_v, gmax=0.2, gstrong=8.0):
    """g and gv ~ U[-gmax, 0), with U[-gstrong, 0) on the token ranges strong_k (key gate)
    and strong_v (value gate); bf16 words."""
    rng = np.random.default_rng(w.seed + 1000)
    B, T, H = w.batch, w.seqlen, w.num_heads
    g = (-gmax * rng.random((B, T, H, w.dk))).astype(np.float32)
    gv = (-gmax * rng.random((B, T, H, w.dv))).astype(np.float32)
    a, b = strong_k
    g[:, a:b] = (-gstrong * rng.random((B, b - a, H, w.dk))).astype(np.float32)
    a, b = strong_v
    gv[:, a:b] = (-gstrong * rng.random((B, b - a, H, w.dv))).astype(np.float32)
    return {"g": inputs.bf16_words(g), "gk": None, "gv": inputs.bf16_words(gv)}


@pytest.mark.parametrize("reverse", [False, True])
def test_gated_bf16_mixed_exact_and_fast_chunks(reverse):
    """Strong decays on some token ranges only, so chunks switch between the exact and the
    fast path (the chunk flags cycle through their slots), on the key side and the value side."""
    w = inputs.Workload("gated_mixed", 2, 400, 4, 4, 128, 128, "bf16", 4, 12, init_std=0.3, seed=70)
    data = w.make()
    gates = _banded_gates(w, (40, 72), (200, 216))
    o, fs, o_ref, fs_ref = _run(w, data, gates, use_gg=False, reverse=reverse)
    tag = " rev" if reverse else ""
    check_fwd(o.cpu().numpy(), fs.cpu().numpy(), o_ref, fs_ref, TOL["bf16"], f"gated_mixed{tag}")


@pytest.mark.parametrize("reverse", [False, True])
def test_gated_bf16_per_channel_rates(reverse):
    """Key channels with very different decay rates (about 0, 0.25 and 1.25 per token on
    average, the last close to the fast path's span per chunk): the rows' log-scales
    drift apart, some rows go back to scale one at almost every chunk, others only with
    the rest; initial state, GQA and g_gamma on."""
    w = inputs.Workload("gated_rates", 2, 1500, 4, 2, 128, 128, "bf16", 5, 12, reverse=reverse, init_std=0.5,
                        seed=71)
    data = w.make()
    rng = np.random.default_rng(w.seed + 2000)
    rate = np.array([0.01, 0.5, 2.5, 0.01])[np.arange(w.dk) % 4].astype(np.float32)
    g = (-rate * rng.random((w.batch, w.seqlen, w.num_heads, w.dk))).astype(np.float32)
    gates = {"g": inputs.bf16_words(g), "gk": None, "gv": None}
    o, fs, o_ref, fs_ref = _run(w, data, gates, use_gg=True, reverse=reverse)
    check_fwd(o.cpu().numpy(), fs.cpu().numpy(), o_ref, fs_ref, TOL["bf16"],
              f"gated_rates{' rev' if reverse else ''}")


@pytest.mark.parametrize("dk", [32, 64, 128])
@pytest.mark.parametrize("which", [("g",), ("g", "gk"), ("gv",), ("g", "gk", "gv")])
def test_gated_bf16_instances(dk, which):
    """Every bf16 kernel instance (summed fp32 key gate or not, value gate or not) at each
    dk: the launch picks the instance from the gates given."""
    w = inputs.Workload(f"gated_inst_dk{dk}", 2, 90, 4, 2, dk, 64, "bf16", 7, 12, init_std=0.3, seed=80 + dk)
    _compare(w, which, gmax=0.6, tag=f" dk{dk} {'+'.join(which)}")

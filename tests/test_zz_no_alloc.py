"""lattn_fwd_noalloc (the forward whose workspace is the library's own device array)
against lattn_fwd with a caller-owned workspace, through the C ABI.

Both run the same kernels in the same order, so the outputs must be bit-identical; one
case is also held to the oracle's bar.  Each case makes two calls in a row on the shared
array, the second with a smaller input, so that stale contents from the first call
would show."""
import ctypes

import pytest

from decayed_recurrent_attention_amd import inputs, lattn
from tests.parity_util import TOL, check_fwd, oracle_run, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lattn.load_library()


def _problem(w):
    return lattn.LattnProblem(w.batch, w.seqlen, w.num_heads, w.num_kv_heads, w.dk, w.dv,
                              w.num_seqs if w.seq_lens is not None else 0,
                              lattn.LATTN_BF16 if w.dtype == "bf16" else lattn.LATTN_F32, lattn.LATTN_F32)


def _both(w, data):
    """(o, final_state) from lattn_fwd with its own workspace and from lattn_fwd_noalloc."""
    import torch

    print(f"[no_alloc] {w.name}: B{w.batch} T{w.seqlen} H{w.num_heads}/{w.num_kv_heads} d{w.dk}x{w.dv}",
          flush=True)
    prob = _problem(w)
    q, k, v = (to_device(data[n], w.dtype) for n in ("q", "k", "v"))
    init = to_device(data["initial_state"], "f32")
    cu = None if data["cu_seqlens"] is None else torch.from_numpy(data["cu_seqlens"]).cuda().to(torch.int32)
    g = torch.from_numpy(lattn.lattn_lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers)).cuda()
    need = lattn.lattn_fwd_workspace_size(prob)
    assert 0 < need <= lattn.LATTN_NOALLOC_SCRATCH_BYTES, need  # the case uses the array
    outs = []
    for noalloc in (False, True):
        o = torch.full((w.batch, w.seqlen, w.num_heads, w.dv), float("nan"), device="cuda")
        fs = torch.full((w.num_seqs, w.num_heads, w.dk, w.dv), float("nan"), device="cuda")
        if noalloc:
            rc = lattn.lattn_fwd_noalloc(prob, q, k, v, g, w.scale, init, w.reverse, cu, o, fs)
        else:
            ws = torch.empty(need, device="cuda", dtype=torch.uint8)
            rc = lattn.lattn_fwd(prob, q, k, v, g, w.scale, init, w.reverse, cu, o, fs, ws)
        assert rc == lattn.LATTN_OK, lattn.lattn_status_string(rc)
        torch.cuda.synchronize()
        outs.append((o, fs))
    return outs


def _same(w, data):
    import torch

    (o1, f1), (o2, f2) = _both(w, data)
    assert torch.equal(o1, o2), f"{w.name}: o differs"
    assert torch.equal(f1, f2), f"{w.name}: final_state differs"
    return o2, f2


def test_packed_twice_second_smaller():
    big = inputs.varlen_gqa(num_seqs=12, lo=64, hi=2000, seed=71)
    small = inputs.varlen_gqa(num_seqs=5, lo=1, hi=300, seed=72, reverse=True)
    _same(big, big.make())
    data = small.make()
    o, fs = _same(small, data)
    o_ref, fs_ref = oracle_run(small, data)
    check_fwd(o.cpu().numpy(), fs.cpu().numpy(), o_ref, fs_ref, TOL["bf16"], "noalloc packed", cu=data["cu_seqlens"])


def test_split_twice_second_smaller():
    big = inputs.Workload("noalloc_split_big", 1, 16384, 4, 4, 128, 128, "bf16", 2, 12, init_std=0.2, seed=73)
    small = inputs.Workload("noalloc_split_small", 1, 3000, 2, 2, 64, 64, "bf16", 4, 12, reverse=True,
                            init_std=0.3, seed=74)
    _same(big, big.make())
    data = small.make()
    o, fs = _same(small, data)
    o_ref, fs_ref = oracle_run(small, data)
    check_fwd(o.cpu().numpy(), fs.cpu().numpy(), o_ref, fs_ref, TOL["bf16"], "noalloc split")


def test_too_large_refused_and_no_workspace_case():
    import torch

    # a forced 64-way split of B1 H8 d256 x 256 needs 2 * 64 * 8 * 256 * 256 * 4 B = 256 MiB
    prob = lattn.LattnProblem(1, 64 * 64, 8, 8, 256, 256, 0, lattn.LATTN_BF16, lattn.LATTN_F32)
    with lattn.knob(lattn.LATTN_KNOB_SPLIT, 64):
        assert lattn.lattn_fwd_workspace_size(prob) > lattn.LATTN_NOALLOC_SCRATCH_BYTES
        fake = 1 << 20  # never dereferenced: the size check comes first
        rc = lattn.load_library().lattn_fwd_noalloc(ctypes.byref(prob), fake, fake, fake, fake, 1.0, None, 0,
                                                    None, fake, fake, None)
        assert rc == lattn.LATTN_ERR_WORKSPACE
    # fixed length without a split needs no workspace: same results as lattn_fwd
    w = inputs.Workload("noalloc_plain", 4, 300, 32, 32, 64, 64, "bf16", 1, 12, seed=75)  # 128 workgroups: no split
    data = w.make()
    prob = _problem(w)
    assert lattn.lattn_fwd_workspace_size(prob) == 0
    q, k, v = (to_device(data[n], w.dtype) for n in ("q", "k", "v"))
    g = torch.from_numpy(lattn.lattn_lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers)).cuda()
    res = []
    for fn in (lattn.lattn_fwd, lattn.lattn_fwd_noalloc):
        o = torch.empty((w.batch, w.seqlen, w.num_heads, w.dv), device="cuda")
        fs = torch.empty((w.batch, w.num_heads, w.dk, w.dv), device="cuda")
        assert fn(prob, q, k, v, g, w.scale, None, False, None, o, fs) == lattn.LATTN_OK
        res.append((o, fs))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])

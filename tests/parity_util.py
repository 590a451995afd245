"""Helpers shared by the GPU parity tests: move seeded inputs to the device, run the
HIP path through its binding, run the oracle, compare with the stated tolerance.

Tolerance (stated for both o and final_state, each over the whole tensor):
    max |gpu - oracle| <= tol * RMS(oracle),  tol = 1e-4 (fp32 inputs), 2e-2 (bf16 inputs).
"""
from __future__ import annotations

import numpy as np

import oracle
from decayed_recurrent_attention_amd import inputs, lattn

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_device(a: np.ndarray | None, dtype: str):
    import torch

    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_run(w: inputs.Workload, data: dict, reverse: bool | None = None, g_gamma=None):
    """Run the HIP path; returns device tensors (o, final_state)."""
    rev = w.reverse if reverse is None else reverse
    q, k, v = (to_device(data[n], w.dtype) for n in ("q", "k", "v"))
    init = to_device(data["initial_state"], "f32")
    cu = data["cu_seqlens"]
    if g_gamma is None:
        return lattn.lightning_attn(q, k, v, w.layer_idx, w.num_layers, softmax_scale=w.scale,
                                    initial_state=init, reverse=rev, cu_seqlens=cu)
    return lattn.recurrent(q, k, v, g_gamma=g_gamma, softmax_scale=w.scale, initial_state=init,
                           reverse=rev, cu_seqlens=cu)


def oracle_run(w: inputs.Workload, data: dict, reverse: bool | None = None, pairs=None,
               g_gamma=None):
    rev = w.reverse if reverse is None else reverse
    orc = oracle.load()
    g = orc.lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers) if g_gamma is None else g_gamma
    return orc.recurrent_fwd(data["q"], data["k"], data["v"], g, w.scale,
                             initial_state=data["initial_state"], reverse=rev,
                             cu_seqlens=data["cu_seqlens"], pairs=pairs)


def gpu_run_bwd(w: inputs.Workload, data: dict, grads: dict, reverse: bool | None = None,
                g_gamma=None, want_d_init: bool = True):
    """Run the HIP backward; returns device tensors (dq, dk, dv, d_initial_state)."""
    import torch

    rev = w.reverse if reverse is None else reverse
    q, k, v = (to_device(data[n], w.dtype) for n in ("q", "k", "v"))
    init = to_device(data["initial_state"], "f32")
    d_o = to_device(grads["d_o"], w.dtype)
    d_fin = to_device(grads["d_final_state"], "f32")
    g = g_gamma
    if g is None:
        g = torch.from_numpy(lattn.lattn_lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers)).cuda()
    return lattn.recurrent_bwd(q, k, v, d_o, g_gamma=g, softmax_scale=w.scale, initial_state=init,
                               d_final_state=d_fin, reverse=rev, cu_seqlens=data["cu_seqlens"],
                               want_d_initial_state=want_d_init)


def oracle_run_bwd(w: inputs.Workload, data: dict, grads: dict, reverse: bool | None = None,
                   g_gamma=None):
    rev = w.reverse if reverse is None else reverse
    orc = oracle.load()
    g = orc.lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers) if g_gamma is None else g_gamma
    return orc.recurrent_bwd(data["q"], data["k"], data["v"], g, w.scale, grads["d_o"],
                             grads["d_final_state"], data["initial_state"], reverse=rev,
                             cu_seqlens=data["cu_seqlens"])


def rel_err(got, ref) -> float:
    """max |got - ref| / RMS(ref) (0 for empty or all-zero references)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.isfinite(got).all(), "non-finite values in the GPU result"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref)))
    if rms == 0.0:
        return 0.0 if err == 0.0 else float("inf")
    return err / rms


def check(got, ref, tol: float, what: str) -> float:
    r = rel_err(got, ref)
    print(f"[parity] {what}: max|err|/RMS = {r:.3e} (tol {tol:.0e})", flush=True)
    assert r <= tol, f"{what}: max|err|/RMS = {r:.3e} exceeds {tol:.0e}"
    return r

"""Helpers shared by the GPU parity tests: move seeded inputs to the device, run the
HIP path through its binding, run the oracle, compare with the stated tolerance.

Tolerance, for every output tensor separately (o, final_state, each gradient):
    max |gpu - oracle| <= tol * RMS(oracle),  tol = 1e-4 (fp32 inputs), 2e-2 (bf16 inputs),
taken twice: over the whole tensor, and over every (sequence, head) slice of it against
that slice's own RMS.  The second bar keeps a fast-decaying head (small outputs) from
being judged against the scale of an undecayed one (outputs growing with t).  The
outputs are float32, so a slice whose exact values lie below float32's normal range
(say lam * D with lam = exp(-200), about 1e-87) cannot be represented at all: the
bars allow an absolute FLT_MIN (2^-126) on top of tol * RMS.
"""
from __future__ import annotations

import numpy as np

import oracle
from decayed_recurrent_attention_amd import inputs, lattn

TOL = {"f32": 1e-4, "bf16": 2e-2}
FLT_MIN = 2.0 ** -126  # smallest normal float32


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


def gpu_run_gated(w: inputs.Workload, data: dict, gates: dict, use_gg: bool = True, reverse: bool | None = None):
    """Run the HIP gated forward with the gates given (None: absent) and, when use_gg,
    the Lightning g_gamma of the workload's layer; returns device tensors (o, final_state)."""
    import torch

    rev = w.reverse if reverse is None else reverse
    gg = lattn.lattn_lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers) if use_gg else None
    dev = {n: to_device(data[n], w.dtype) for n in ("q", "k", "v")}
    gd = {n: to_device(x, w.dtype) for n, x in gates.items() if x is not None}
    return lattn.recurrent_gated(dev["q"], dev["k"], dev["v"], **gd,
                                 g_gamma=None if gg is None else torch.from_numpy(gg).cuda(),
                                 softmax_scale=w.scale, initial_state=to_device(data["initial_state"], "f32"),
                                 reverse=rev, cu_seqlens=data["cu_seqlens"])


def oracle_run_gated(w: inputs.Workload, data: dict, gates: dict, use_gg: bool = True,
                     reverse: bool | None = None):
    rev = w.reverse if reverse is None else reverse
    orc = oracle.load()
    gg = orc.lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers) if use_gg else None
    return orc.recurrent_gated_fwd(data["q"], data["k"], data["v"], **gates, g_gamma=gg, scale=w.scale,
                                   initial_state=data["initial_state"], reverse=rev,
                                   cu_seqlens=data["cu_seqlens"])


class Accum:
    """Streaming parity statistics of one output tensor: the whole-tensor maximum error
    and sum of squares, and the same per (sequence, head) slice.  Feed it pieces of the
    tensor with `add_*`; `finish` applies both bars."""

    def __init__(self, what: str):
        self.what = what
        self.err = 0.0
        self.ss = 0.0
        self.count = 0
        self.slices: dict = {}  # (sequence, head) -> [max err, sum of squares, count]

    def _add(self, key, diff_max, ss, count):
        s = self.slices.setdefault(key, [0.0, 0.0, 0])
        s[0] = max(s[0], diff_max)
        s[1] += ss
        s[2] += count

    def add(self, got, ref, axes_keep, key_of):
        """got, ref: equal-shape arrays.  The slices are indexed by the axes `axes_keep`
        (two of them); key_of maps their index pair to a (sequence, head) key."""
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert got.shape == ref.shape, (self.what, got.shape, ref.shape)
        if ref.size == 0:
            return
        assert np.isfinite(got).all(), f"{self.what}: non-finite values in the GPU result"
        red = tuple(a for a in range(ref.ndim) if a not in axes_keep)
        diff = np.abs(got - ref)
        dmax = diff.max(axis=red)
        ss = np.square(ref).sum(axis=red)
        cnt = ref.size // (dmax.size or 1)
        self.err = max(self.err, float(dmax.max()))
        self.ss += float(ss.sum())
        self.count += ref.size
        for i in range(dmax.shape[0]):
            for j in range(dmax.shape[1]):
                self._add(key_of(i, j), float(dmax[i, j]), float(ss[i, j]), cnt)

    def add_tokens(self, got, ref, cu=None, row0: int = 0):
        """[B, T, H, d] token outputs (o, dq, dk, dv); slices are (batch row, head), or
        (packed sequence, head) with cu_seqlens.  row0 offsets the batch-row index of a
        piece cut from a larger tensor."""
        if cu is None:
            self.add(got, ref, (0, 2), lambda i, j: (row0 + i, j))
            return
        cu = np.asarray(cu, dtype=np.int64)
        for n in range(len(cu) - 1):
            a, b = int(cu[n]), int(cu[n + 1])
            if b > a:
                self.add(got[:, a:b], ref[:, a:b], (0, 2), lambda i, j, n=n: (n, j))

    def add_states(self, got, ref, n0: int = 0):
        """[N, H, dk, dv] states; slices are (sequence, head)."""
        self.add(got, ref, (0, 1), lambda i, j: (n0 + i, j))

    def add_rows(self, got, ref):
        """[B, H, d] per-sequence vectors (decode o); slices are (batch row, head)."""
        got = np.asarray(got)[:, None]
        ref = np.asarray(ref)[:, None]
        self.add(got, ref, (0, 2), lambda i, j: (i, j))

    def finish(self, tol: float, per_slice_tol: float | None = None) -> float:
        """Assert the whole-tensor bar and the per-slice bar; return the whole-tensor ratio."""
        pt = tol if per_slice_tol is None else per_slice_tol
        rms = np.sqrt(self.ss / self.count) if self.count else 0.0
        e_whole = max(0.0, self.err - FLT_MIN)
        whole = 0.0 if self.count == 0 else (e_whole / rms if rms > 0 else (0.0 if e_whole == 0 else np.inf))
        worst, worst_key = 0.0, None
        for key, (e, ss, c) in self.slices.items():
            r = np.sqrt(ss / c) if c else 0.0
            e = max(0.0, e - FLT_MIN)  # below float32's normal range nothing is representable
            ratio = e / r if r > 0 else (0.0 if e == 0 else np.inf)
            if ratio >= worst:
                worst, worst_key = ratio, key
        print(f"[parity] {self.what}: max|err|/RMS = {whole:.3e} whole tensor, {worst:.3e} worst "
              f"(sequence, head) slice {worst_key} of {len(self.slices)} (tol {tol:.0e})", flush=True)
        assert whole <= tol, f"{self.what}: max|err|/RMS = {whole:.3e} exceeds {tol:.0e}"
        assert worst <= pt, (f"{self.what}: slice {worst_key} max|err|/RMS(slice) = {worst:.3e} "
                             f"exceeds {pt:.0e}")
        return whole


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


def check(got, ref, tol: float, what: str, kind: str = "tokens", cu=None) -> float:
    """Both bars (whole tensor and per (sequence, head) slice) on one output.

    kind: "tokens" for [B, T, H, d] outputs (cu: the packed sequence bounds, if any),
    "states" for [N, H, dk, dv], "rows" for [B, H, d]."""
    acc = Accum(what)
    if kind == "tokens":
        acc.add_tokens(got, ref, cu)
    elif kind == "states":
        acc.add_states(got, ref)
    elif kind == "rows":
        acc.add_rows(got, ref)
    else:
        raise ValueError(kind)
    return acc.finish(tol)


def check_fwd(o, fs, o_ref, fs_ref, tol: float, what: str, cu=None):
    """o and final_state of one forward call against the oracle."""
    check(o, o_ref, tol, what + " o", "tokens", cu)
    check(fs, fs_ref, tol, what + " final_state", "states")

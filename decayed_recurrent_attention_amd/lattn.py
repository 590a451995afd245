"""Python binding of liblattn.so (the C ABI in include/lattn.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the forward pass runs in the library's kernels.  A
missing library raises; there is no fallback path.

Functions with the C names (``lattn_fwd``, ``lattn_bwd`` and their workspace
queries, ``lattn_lightning_g_gamma``, ``lattn_status_string``) map one to one onto
the ABI.  ``lightning_attn`` and ``recurrent`` mirror the signatures of the ejkernel
lightning_attn and recurrent interface pages (without the GLA gates);
``recurrent_bwd`` and ``lightning_attn_bwd`` return the gradients of those.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblattn.so")

LATTN_BF16 = 0
LATTN_F32 = 1

LATTN_OK = 0
LATTN_ERR_INVALID_ARG = -1
LATTN_ERR_VARLEN_BATCH = -2
LATTN_ERR_HEADS = -3
LATTN_ERR_UNSUPPORTED = -4
LATTN_ERR_WORKSPACE = -5
LATTN_ERR_LAUNCH = -6
LATTN_ERR_DEVICE = -7

# Every function declared in include/lattn.h.
EXPORTS = ("lattn_fwd", "lattn_fwd_noalloc", "lattn_fwd_workspace_size", "lattn_fwd_gated", "lattn_fwd_gated_workspace_size",
           "lattn_bwd", "lattn_bwd_workspace_size", "lattn_decode", "lattn_lightning_g_gamma",
           "lattn_status_string", "lattn_set_knob", "lattn_abi_version")

# Knobs of lattn_set_knob (forced kernel choices for tests and measurements).
LATTN_KNOB_AUTO = -1
LATTN_KNOB_WAVES = 0
LATTN_KNOB_SPLIT = 1
LATTN_KNOB_BWD_PAIR = 2


class LattnProblem(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "seqlen", "num_heads", "num_kv_heads", "head_dim_qk", "head_dim_v",
        "num_seqs", "in_dtype", "out_dtype")]


class LattnError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"lattn status {status}: {lattn_status_string(status)}")
        self.status = status


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblattn.so once (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is missing: build it with "
                                   "`python -m decayed_recurrent_attention_amd.build`")
            lib = ctypes.CDLL(path)
            P = ctypes.POINTER(LattnProblem)
            vp = ctypes.c_void_p
            lib.lattn_fwd.restype = ctypes.c_int
            lib.lattn_fwd.argtypes = [P, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_int, vp, vp,
                                      vp, vp, ctypes.c_size_t, vp]
            lib.lattn_fwd_noalloc.restype = ctypes.c_int
            lib.lattn_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_int, vp, vp, vp, vp]
            lib.lattn_fwd_workspace_size.restype = ctypes.c_size_t
            lib.lattn_fwd_workspace_size.argtypes = [P]
            lib.lattn_bwd.restype = ctypes.c_int
            lib.lattn_bwd.argtypes = [P, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_int, vp, vp, vp,
                                      vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
            lib.lattn_bwd_workspace_size.restype = ctypes.c_size_t
            lib.lattn_bwd_workspace_size.argtypes = [P]
            lib.lattn_fwd_gated.restype = ctypes.c_int
            lib.lattn_fwd_gated.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_int, vp,
                                            vp, vp, vp, ctypes.c_size_t, vp]
            lib.lattn_fwd_gated_workspace_size.restype = ctypes.c_size_t
            lib.lattn_fwd_gated_workspace_size.argtypes = [P, ctypes.c_int]
            lib.lattn_decode.restype = ctypes.c_int
            lib.lattn_decode.argtypes = [P, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp]
            lib.lattn_lightning_g_gamma.restype = ctypes.c_int
            lib.lattn_lightning_g_gamma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
            lib.lattn_status_string.restype = ctypes.c_char_p
            lib.lattn_status_string.argtypes = [ctypes.c_int]
            lib.lattn_set_knob.restype = ctypes.c_int
            lib.lattn_set_knob.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
            lib.lattn_abi_version.restype = ctypes.c_int
            lib.lattn_abi_version.argtypes = []
            _lib = lib
    return _lib


# -- one-to-one ABI wrappers ------------------------------------------------------
def lattn_status_string(status: int) -> str:
    return load_library().lattn_status_string(int(status)).decode()


def lattn_abi_version() -> int:
    return int(load_library().lattn_abi_version())


def lattn_set_knob(which: int, value: int) -> int:
    """Force a kernel choice (LATTN_KNOB_AUTO restores the automatic one); returns the
    knob's previous value."""
    prev = ctypes.c_int(0)
    rc = load_library().lattn_set_knob(int(which), int(value), ctypes.byref(prev))
    if rc != LATTN_OK:
        raise LattnError(rc)
    return prev.value


@contextlib.contextmanager
def knob(which: int, value: int):
    """Context manager: the knob holds `value` inside the block, its old value after."""
    prev = lattn_set_knob(which, value)
    try:
        yield
    finally:
        lattn_set_knob(which, prev)


def lattn_fwd_workspace_size(problem: LattnProblem) -> int:
    return int(load_library().lattn_fwd_workspace_size(ctypes.byref(problem)))


def lattn_bwd_workspace_size(problem: LattnProblem) -> int:
    return int(load_library().lattn_bwd_workspace_size(ctypes.byref(problem)))


def lattn_lightning_g_gamma(num_heads: int, layer_idx: int, num_layers: int) -> np.ndarray:
    """Lightning per-head log-decay as float32 [num_heads] (host)."""
    out = np.empty(num_heads, dtype=np.float32)
    rc = load_library().lattn_lightning_g_gamma(int(num_heads), int(layer_idx), int(num_layers),
                                                out.ctypes.data)
    if rc != LATTN_OK:
        raise LattnError(rc)
    return out


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr()) or None


def lattn_fwd(problem: LattnProblem, q, k, v, g_gamma, scale: float, initial_state, reverse: bool,
              cu_seqlens, o, final_state, workspace=None, stream=None) -> int:
    """Raw call: tensors (or None) are passed by address; returns the status code."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return int(load_library().lattn_fwd(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(g_gamma), float(scale),
        _ptr(initial_state), int(bool(reverse)), _ptr(cu_seqlens), _ptr(o), _ptr(final_state),
        _ptr(workspace), ws_bytes, stream))


LATTN_NOALLOC_SCRATCH_BYTES = 32 << 20


def lattn_fwd_noalloc(problem: LattnProblem, q, k, v, g_gamma, scale: float, initial_state, reverse: bool,
                      cu_seqlens, o, final_state, stream=None) -> int:
    """Raw call of the forward that takes its workspace from the library's own device
    array (nothing is allocated); returns the status code."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().lattn_fwd_noalloc(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(g_gamma), float(scale),
        _ptr(initial_state), int(bool(reverse)), _ptr(cu_seqlens), _ptr(o), _ptr(final_state), stream))


def lattn_bwd(problem: LattnProblem, q, k, v, g_gamma, scale: float, initial_state, reverse: bool,
              cu_seqlens, d_o, d_final_state, dq, dk, dv, d_initial_state, workspace=None,
              stream=None) -> int:
    """Raw call: tensors (or None) are passed by address; returns the status code."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return int(load_library().lattn_bwd(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(g_gamma), float(scale),
        _ptr(initial_state), int(bool(reverse)), _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final_state),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(d_initial_state), _ptr(workspace), ws_bytes, stream))


LATTN_GATE_G, LATTN_GATE_GK, LATTN_GATE_GV = 1, 2, 4


def lattn_fwd_gated_workspace_size(problem: LattnProblem, gates: int) -> int:
    return int(load_library().lattn_fwd_gated_workspace_size(ctypes.byref(problem), int(gates)))


def lattn_fwd_gated(problem: LattnProblem, q, k, v, g, gk, gv, g_gamma, scale: float, initial_state,
                    reverse: bool, cu_seqlens, o, final_state, workspace=None, stream=None) -> int:
    """Raw call: tensors (or None) are passed by address; returns the status code."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return int(load_library().lattn_fwd_gated(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gk), _ptr(gv), _ptr(g_gamma),
        float(scale), _ptr(initial_state), int(bool(reverse)), _ptr(cu_seqlens), _ptr(o),
        _ptr(final_state), _ptr(workspace), ws_bytes, stream))


def lattn_decode(problem: LattnProblem, q, k, v, g_gamma, scale: float, state_in, state_out, o,
                 stream=None) -> int:
    """Raw call: tensors (or None) are passed by address; returns the status code."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().lattn_decode(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(g_gamma), float(scale), _ptr(state_in),
        _ptr(state_out), _ptr(o), stream))


# -- tensor-level forward and backward ----------------------------------------------
_G_CACHE: dict = {}


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return LATTN_BF16
    if t.dtype == torch.float32:
        return LATTN_F32
    raise TypeError(f"q, k, v must be bfloat16 or float32, got {t.dtype}")


class _Args:
    """Validated, contiguous arguments shared by the forward and backward calls."""


def _prepare(query, key, value, g_gamma, softmax_scale, initial_state, cu_seqlens) -> _Args:
    import torch

    a = _Args()
    a.squeeze = query.dim() == 3
    if a.squeeze:
        if cu_seqlens is None:
            raise ValueError("3-D inputs are only accepted with cu_seqlens")
        query, key, value = query.unsqueeze(0), key.unsqueeze(0), value.unsqueeze(0)
    if query.dim() != 4 or key.dim() != 4 or value.dim() != 4:
        raise ValueError("query, key and value must be 4-D (batch, seq, heads, dim)")
    B, T, H, dk = query.shape
    Hkv = key.shape[2]
    dv = value.shape[3]
    if key.shape != (B, T, Hkv, dk) or value.shape != (B, T, Hkv, dv):
        raise ValueError(f"inconsistent shapes q{tuple(query.shape)} k{tuple(key.shape)} "
                         f"v{tuple(value.shape)}")
    if not (query.dtype == key.dtype == value.dtype):
        raise TypeError("query, key and value must share one dtype")
    dev = query.device
    if dev.type != "cuda":
        raise ValueError("inputs must be GPU tensors")
    num_seqs = 0
    cu = None
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError(f"cu_seqlens needs batch size 1 (got {B}); pack the sequences "
                             "along the token axis")
        cu = torch.as_tensor(cu_seqlens).to(device=dev, dtype=torch.int32).contiguous()
        num_seqs = cu.numel() - 1
        if num_seqs < 1:
            raise ValueError("cu_seqlens needs at least two entries")
        if initial_state is not None and initial_state.shape[0] != num_seqs:
            raise ValueError(f"initial_state holds {initial_state.shape[0]} states but "
                             f"cu_seqlens describes {num_seqs} sequences")
    a.n_seq = num_seqs if cu is not None else B
    if softmax_scale is None:
        softmax_scale = float(np.float32(dk ** -0.5))
    if g_gamma is None:
        g_gamma = torch.zeros(H, device=dev, dtype=torch.float32)
    g_gamma = torch.as_tensor(g_gamma).to(device=dev, dtype=torch.float32).contiguous()
    if g_gamma.shape != (H,):
        raise ValueError(f"g_gamma must have shape ({H},)")
    a.state_shape = (a.n_seq, H, dk, dv)
    if initial_state is not None:
        initial_state = initial_state.to(device=dev, dtype=torch.float32).contiguous()
        if initial_state.shape != a.state_shape:
            raise ValueError(f"initial_state must have shape {a.state_shape}")
    a.q, a.k, a.v = query.contiguous(), key.contiguous(), value.contiguous()
    a.cu, a.g, a.scale, a.init, a.dev = cu, g_gamma, softmax_scale, initial_state, dev
    a.B, a.T, a.H, a.Hkv, a.dk, a.dv = B, T, H, Hkv, dk, dv
    a.prob = LattnProblem(B, T, H, Hkv, dk, dv, num_seqs, _dtype_code(a.q), LATTN_F32)
    return a


def recurrent(query, key, value, g=None, g_gamma=None, gk=None, gv=None, softmax_scale=None,
              initial_state=None, reverse=False, cu_seqlens=None, out_dtype=None):
    """Decayed recurrent attention forward on the GPU (the recurrent interface page's
    argument order).

    Shapes follow that page: q [B, T, H, dk], k [B, T, Hkv, dk], v [B, T, Hkv, dv];
    packed input (``cu_seqlens``) may drop the batch axis.  g, gk ([.., T, H, dk]) and gv
    ([.., T, H, dv]) are optional per-token log-decay gates in the dtype of q; with any
    of them the gated kernel runs, else the Lightning kernel with g_gamma [H].
    Returns (o [.., T, H, dv], final_state float32 [N_seq, H, dk, dv]); o is float32, or
    bf16 with ``out_dtype=torch.bfloat16`` for bf16 input without gates (each element the
    round-to-nearest-even of the float32 result).
    """
    import torch

    bf16_out = out_dtype is not None and out_dtype == torch.bfloat16
    if out_dtype is not None and out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    if g is not None or gk is not None or gv is not None:
        if bf16_out:
            raise ValueError("the gated recurrence returns o in float32 only")
        return recurrent_gated(query, key, value, g=g, gk=gk, gv=gv, g_gamma=g_gamma,
                               softmax_scale=softmax_scale, initial_state=initial_state,
                               reverse=reverse, cu_seqlens=cu_seqlens)
    a = _prepare(query, key, value, g_gamma, softmax_scale, initial_state, cu_seqlens)
    if bf16_out:
        if a.q.dtype != torch.bfloat16:
            raise ValueError("a bf16 o needs bf16 inputs")
        a.prob.out_dtype = LATTN_BF16
    o = torch.empty((a.B, a.T, a.H, a.dv), device=a.dev,
                    dtype=torch.bfloat16 if bf16_out else torch.float32)
    fs = torch.empty(a.state_shape, device=a.dev, dtype=torch.float32)
    ws_bytes = lattn_fwd_workspace_size(a.prob)
    ws = torch.empty(ws_bytes, device=a.dev, dtype=torch.uint8) if ws_bytes else None
    rc = lattn_fwd(a.prob, a.q, a.k, a.v, a.g, a.scale, a.init, reverse, a.cu, o, fs, ws)
    if rc != LATTN_OK:
        raise LattnError(rc)
    return (o[0] if a.squeeze else o), fs


def recurrent_gated(query, key, value, g=None, gk=None, gv=None, g_gamma=None, softmax_scale=None,
                    initial_state=None, reverse=False, cu_seqlens=None):
    """Forward with per-token log-decay gates (gated kernel; see lattn_fwd_gated)."""
    import torch

    a = _prepare(query, key, value, g_gamma, softmax_scale, initial_state, cu_seqlens)
    gates = []
    for name, x, d in (("g", g, a.dk), ("gk", gk, a.dk), ("gv", gv, a.dv)):
        if x is not None:
            if a.squeeze:
                x = x.unsqueeze(0)
            if x.dtype != a.q.dtype:
                raise TypeError(f"{name} must have the dtype of the inputs ({a.q.dtype}), got {x.dtype}")
            x = x.to(device=a.dev).contiguous()
            if x.shape != (a.B, a.T, a.H, d):
                raise ValueError(f"{name} must have shape {(a.B, a.T, a.H, d)}")
        gates.append(x)
    o = torch.empty((a.B, a.T, a.H, a.dv), device=a.dev, dtype=torch.float32)
    fs = torch.empty(a.state_shape, device=a.dev, dtype=torch.float32)
    mask = sum(bit for bit, x in zip((LATTN_GATE_G, LATTN_GATE_GK, LATTN_GATE_GV), gates) if x is not None)
    ws_bytes = lattn_fwd_gated_workspace_size(a.prob, mask)
    ws = torch.empty(ws_bytes, device=a.dev, dtype=torch.uint8) if ws_bytes else None
    g_gamma_t = None if g_gamma is None else a.g
    rc = lattn_fwd_gated(a.prob, a.q, a.k, a.v, *gates, g_gamma_t, a.scale, a.init, reverse, a.cu, o, fs, ws)
    if rc != LATTN_OK:
        raise LattnError(rc)
    return (o[0] if a.squeeze else o), fs


def recurrent_gla(query, key, value, g=None, g_gamma=None, softmax_scale=None, initial_state=None,
                  reverse=False, cu_seqlens=None):
    """Gated linear attention (recurrent_gla page): the recurrence with the per-key-channel
    gate g and the per-head decay g_gamma; the default scale is dk^-1/2."""
    if cu_seqlens is not None and query.dim() == 4 and query.shape[0] != 1:
        raise ValueError(f"cu_seqlens needs batch size 1 (got {query.shape[0]}); pack the "
                         "sequences along the token axis")
    if cu_seqlens is not None and initial_state is not None and \
            initial_state.shape[0] != len(cu_seqlens) - 1:
        raise ValueError(f"initial_state holds {initial_state.shape[0]} states but cu_seqlens "
                         f"describes {len(cu_seqlens) - 1} sequences")
    if g is None:
        return recurrent(query, key, value, g_gamma=g_gamma, softmax_scale=softmax_scale,
                         initial_state=initial_state, reverse=reverse, cu_seqlens=cu_seqlens)
    return recurrent_gated(query, key, value, g=g, g_gamma=g_gamma, softmax_scale=softmax_scale,
                           initial_state=initial_state, reverse=reverse, cu_seqlens=cu_seqlens)


def recurrent_bwd(query, key, value, d_o, g_gamma=None, softmax_scale=None, initial_state=None,
                  d_final_state=None, reverse=False, cu_seqlens=None, want_d_initial_state=True):
    """Gradients of ``recurrent`` on the GPU for output gradient ``d_o`` (the shape of
    o, in the dtype of the inputs) and ``d_final_state`` (float32 [N_seq, H, dk, dv]
    or None).

    Returns float32 (dq [.., T, H, dk], dk [.., T, Hkv, dk], dv [.., T, Hkv, dv],
    d_initial_state [N_seq, H, dk, dv] or None).
    """
    import torch

    a = _prepare(query, key, value, g_gamma, softmax_scale, initial_state, cu_seqlens)
    if a.squeeze:
        d_o = d_o.unsqueeze(0)
    if d_o.dtype != a.q.dtype:
        raise TypeError(f"d_o must have the dtype of the inputs ({a.q.dtype}), got {d_o.dtype}")
    d_o = d_o.to(device=a.dev).contiguous()
    if d_o.shape != (a.B, a.T, a.H, a.dv):
        raise ValueError(f"d_o must have shape {(a.B, a.T, a.H, a.dv)}")
    if d_final_state is not None:
        d_final_state = d_final_state.to(device=a.dev, dtype=torch.float32).contiguous()
        if d_final_state.shape != a.state_shape:
            raise ValueError(f"d_final_state must have shape {a.state_shape}")
    f32 = dict(device=a.dev, dtype=torch.float32)
    dq = torch.empty((a.B, a.T, a.H, a.dk), **f32)
    dk = torch.empty((a.B, a.T, a.Hkv, a.dk), **f32)
    dv = torch.empty((a.B, a.T, a.Hkv, a.dv), **f32)
    d_init = torch.empty(a.state_shape, **f32) if want_d_initial_state else None
    ws_bytes = lattn_bwd_workspace_size(a.prob)
    ws = torch.empty(ws_bytes, device=a.dev, dtype=torch.uint8) if ws_bytes else None
    rc = lattn_bwd(a.prob, a.q, a.k, a.v, a.g, a.scale, a.init, reverse, a.cu, d_o, d_final_state,
                   dq, dk, dv, d_init, ws)
    if rc != LATTN_OK:
        raise LattnError(rc)
    if a.squeeze:
        dq, dk, dv = dq[0], dk[0], dv[0]
    return dq, dk, dv, d_init


def lightning_g_gamma_tensor(num_heads: int, layer_idx: int, num_layers: int, device):
    """Device copy of the lightning decay schedule (cached per device and arguments)."""
    import torch

    key = (num_heads, layer_idx, num_layers, str(device))
    g = _G_CACHE.get(key)
    if g is None:
        g = torch.from_numpy(lattn_lightning_g_gamma(num_heads, layer_idx, num_layers)).to(device)
        _G_CACHE[key] = g
    return g


def lightning_attn(query, key, value, layer_idx: int, num_layers: int, softmax_scale=None,
                   initial_state=None, reverse=False, cu_seqlens=None, out_dtype=None):
    """Lightning attention forward (lightning_attn interface page): the layer-dependent
    decay schedule, default scale dk^-1/2, then the recurrent forward."""
    if num_layers < 1 or not 0 <= layer_idx <= num_layers:
        raise ValueError("need num_layers >= 1 and 0 <= layer_idx <= num_layers")
    if cu_seqlens is not None and query.dim() == 4 and query.shape[0] != 1:
        raise ValueError(f"cu_seqlens needs batch size 1 (got {query.shape[0]}); pack the "
                         "sequences along the token axis")
    if cu_seqlens is not None and initial_state is not None and \
            initial_state.shape[0] != len(cu_seqlens) - 1:
        raise ValueError(f"initial_state holds {initial_state.shape[0]} states but cu_seqlens "
                         f"describes {len(cu_seqlens) - 1} sequences")
    if softmax_scale is None:
        softmax_scale = float(np.float32(key.shape[-1] ** -0.5))
    g = lightning_g_gamma_tensor(query.shape[-2], layer_idx, num_layers, query.device)
    return recurrent(query, key, value, g_gamma=g, softmax_scale=softmax_scale,
                     initial_state=initial_state, reverse=reverse, cu_seqlens=cu_seqlens,
                     out_dtype=out_dtype)


def lightning_attn_bwd(query, key, value, d_o, layer_idx: int, num_layers: int, softmax_scale=None,
                       initial_state=None, d_final_state=None, reverse=False, cu_seqlens=None):
    """Gradients of ``lightning_attn`` (same decay schedule and default scale)."""
    if num_layers < 1 or not 0 <= layer_idx <= num_layers:
        raise ValueError("need num_layers >= 1 and 0 <= layer_idx <= num_layers")
    if softmax_scale is None:
        softmax_scale = float(np.float32(key.shape[-1] ** -0.5))
    g = lightning_g_gamma_tensor(query.shape[-2], layer_idx, num_layers, query.device)
    return recurrent_bwd(query, key, value, d_o, g_gamma=g, softmax_scale=softmax_scale,
                         initial_state=initial_state, d_final_state=d_final_state, reverse=reverse,
                         cu_seqlens=cu_seqlens)


def decode_step(query, key, value, state, g_gamma=None, softmax_scale=None, in_place=True):
    """One decoding step: q, k, v of one new token per sequence ([B, H|Hkv, d] or
    [B, 1, H|Hkv, d]) and the float32 state [B, H, dk, dv] (None for zeros).

    Returns (o float32 [B, H, dv] (or [B, 1, H, dv]), new state).  With ``in_place``
    the new state overwrites ``state``.
    """
    import torch

    unsq = query.dim() == 4
    if unsq:
        if query.shape[1] != 1:
            raise ValueError("decode_step takes one token per sequence")
        query, key, value = query[:, 0], key[:, 0], value[:, 0]
    if query.dim() != 3 or key.dim() != 3 or value.dim() != 3:
        raise ValueError("query, key and value must be [batch, heads, dim]")
    B, H, dk = query.shape
    Hkv, dv = key.shape[1], value.shape[2]
    if key.shape != (B, Hkv, dk) or value.shape != (B, Hkv, dv):
        raise ValueError("inconsistent q/k/v shapes")
    if not (query.dtype == key.dtype == value.dtype):
        raise TypeError("query, key and value must share one dtype")
    dev = query.device
    if dev.type != "cuda":
        raise ValueError("inputs must be GPU tensors")
    if softmax_scale is None:
        softmax_scale = float(np.float32(dk ** -0.5))
    if g_gamma is None:
        g_gamma = torch.zeros(H, device=dev, dtype=torch.float32)
    g_gamma = torch.as_tensor(g_gamma).to(device=dev, dtype=torch.float32).contiguous()
    if state is not None:
        if state.shape != (B, H, dk, dv) or state.dtype != torch.float32 or not state.is_contiguous():
            raise ValueError(f"state must be a contiguous float32 tensor of shape {(B, H, dk, dv)}")
    out_state = state if (in_place and state is not None) else torch.empty(
        (B, H, dk, dv), device=dev, dtype=torch.float32)
    q, k, v = query.contiguous(), key.contiguous(), value.contiguous()
    o = torch.empty((B, H, dv), device=dev, dtype=torch.float32)
    prob = LattnProblem(B, 1, H, Hkv, dk, dv, 0, _dtype_code(q), LATTN_F32)
    rc = lattn_decode(prob, q, k, v, g_gamma, softmax_scale, state, out_state, o)
    if rc != LATTN_OK:
        raise LattnError(rc)
    return (o.unsqueeze(1) if unsq else o), out_state

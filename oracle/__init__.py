"""CPU fp64 oracle for decayed recurrent (Lightning) attention, forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library never
imports it, and it imports nothing from the GPU library: the two share no code.

The arithmetic lives in ``lattn_oracle.c`` (plain C, fp64, one token at a time,
following the update equation of the ejkernel ``recurrent`` page).  This module
only marshals numpy arrays into it.

Inputs are numpy arrays in the (batch, seq, heads, dim) layout of the pages.  They
may be ``float32`` (exact values) or ``uint16`` (bf16 words, read exactly).  For
packed variable-length input the leading batch axis may be dropped or be 1.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB, build

__all__ = ["Oracle", "load"]

_IN_BF16 = 0
_IN_F32 = 1


def _in_dtype(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return _IN_BF16
    if a.dtype == np.float32:
        return _IN_F32
    raise TypeError(f"oracle inputs must be float32 values or uint16 bf16 words, got {a.dtype}")


class Oracle:
    """ctypes view of one built oracle library."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_lightning_g_gamma.restype = ctypes.c_int
        lib.oracle_lightning_g_gamma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_void_p]
        lib.oracle_set_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_recurrent_fwd.restype = ctypes.c_int
        lib.oracle_recurrent_fwd.argtypes = (
            [ctypes.c_int] * 7
            + [ctypes.c_void_p] * 4
            + [ctypes.c_double, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        )
        lib.oracle_recurrent_gated_fwd.restype = ctypes.c_int
        lib.oracle_recurrent_gated_fwd.argtypes = (
            [ctypes.c_int] * 7
            + [ctypes.c_void_p] * 7
            + [ctypes.c_double, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
               ctypes.c_void_p, ctypes.c_void_p]
        )
        lib.oracle_recurrent_bwd.restype = ctypes.c_int
        lib.oracle_recurrent_bwd.argtypes = (
            [ctypes.c_int] * 7
            + [ctypes.c_void_p] * 4
            + [ctypes.c_double, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
            + [ctypes.c_void_p] * 6
        )
        self._lib = lib

    # -- decay schedule ---------------------------------------------------------
    def lightning_g_gamma(self, num_heads: int, layer_idx: int, num_layers: int) -> np.ndarray:
        """Per-head log-decay of the lightning_attn wrapper, float32 [num_heads]."""
        out = np.empty(num_heads, dtype=np.float32)
        rc = self._lib.oracle_lightning_g_gamma(num_heads, layer_idx, num_layers,
                                                out.ctypes.data)
        if rc != 0:
            raise ValueError("invalid g_gamma arguments")
        return out

    def set_threads(self, n: int = 0) -> int:
        """Set the OpenMP thread count (n > 0) and return the count in effect."""
        return int(self._lib.oracle_set_threads(int(n)))

    # -- forward recurrence -----------------------------------------------------
    def recurrent_fwd(self, q, k, v, g_gamma, scale, initial_state=None, reverse=False,
                      cu_seqlens=None, pairs=None):
        """Step-by-step fp64 forward.  Returns (o [.., T, H, dv] fp64, final_state fp64).

        ``pairs``: optional iterable of (sequence, head) to compute; outputs of the
        other pairs are NaN.
        """
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        squeeze = q.ndim == 3
        if squeeze:
            q, k, v = q[None], k[None], v[None]
        if not (q.dtype == k.dtype == v.dtype):
            raise TypeError("q, k, v must share one dtype")
        dt = _in_dtype(q)
        B, T, H, dk = q.shape
        Hkv = k.shape[2]
        dv = v.shape[3]
        if k.shape != (B, T, Hkv, dk) or v.shape != (B, T, Hkv, dv):
            raise ValueError("inconsistent q/k/v shapes")
        g = np.ascontiguousarray(g_gamma, dtype=np.float32)
        if g.shape != (H,):
            raise ValueError("g_gamma must have shape [num_heads]")
        if cu_seqlens is not None:
            cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
            n_seq = cu.shape[0] - 1
            cu_ptr = cu.ctypes.data
        else:
            cu = None
            n_seq = B
            cu_ptr = None
        init_ptr = None
        if initial_state is not None:
            init = np.ascontiguousarray(initial_state, dtype=np.float32)
            if init.shape != (n_seq, H, dk, dv):
                raise ValueError(f"initial_state must be {(n_seq, H, dk, dv)}, got {init.shape}")
            init_ptr = init.ctypes.data
        mask_ptr = None
        if pairs is not None:
            mask = np.zeros(n_seq * H, dtype=np.uint8)
            for n, h in pairs:
                mask[n * H + h] = 1
            mask_ptr = mask.ctypes.data
            o = np.full((B, T, H, dv), np.nan)
            fs = np.full((n_seq, H, dk, dv), np.nan)
        else:
            o = np.zeros((B, T, H, dv))
            fs = np.zeros((n_seq, H, dk, dv))
        rc = self._lib.oracle_recurrent_fwd(
            B, T, H, Hkv, dk, dv, dt, q.ctypes.data, k.ctypes.data, v.ctypes.data,
            g.ctypes.data, float(scale), init_ptr, int(bool(reverse)), cu_ptr, n_seq, mask_ptr,
            o.ctypes.data, fs.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return (o[0] if squeeze else o), fs

    # -- gated forward -----------------------------------------------------------
    def recurrent_gated_fwd(self, q, k, v, g=None, gk=None, gv=None, g_gamma=None, scale=1.0,
                            initial_state=None, reverse=False, cu_seqlens=None):
        """fp64 forward with log-decay gates: g, gk [.., T, H, dk] per key channel, gv
        [.., T, H, dv] per value channel (each in the dtype of q, k, v, or None), g_gamma [H]
        float32 or None.  Returns (o, final_state) like recurrent_fwd."""
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        squeeze = q.ndim == 3
        gates = [None if x is None else np.ascontiguousarray(x) for x in (g, gk, gv)]
        if squeeze:
            q, k, v = q[None], k[None], v[None]
            gates = [None if x is None else x[None] for x in gates]
        if not (q.dtype == k.dtype == v.dtype):
            raise TypeError("q, k, v must share one dtype")
        dt = _in_dtype(q)
        B, T, H, dk = q.shape
        Hkv = k.shape[2]
        dv = v.shape[3]
        if k.shape != (B, T, Hkv, dk) or v.shape != (B, T, Hkv, dv):
            raise ValueError("inconsistent q/k/v shapes")
        for x, d in zip(gates, (dk, dk, dv)):
            if x is not None and (x.dtype != q.dtype or x.shape != (B, T, H, d)):
                raise ValueError("gates need the dtype of q and shape [B, T, H, dk | dv]")
        gg = None if g_gamma is None else np.ascontiguousarray(g_gamma, dtype=np.float32)
        if cu_seqlens is not None:
            cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
            n_seq = cu.shape[0] - 1
            cu_ptr = cu.ctypes.data
        else:
            n_seq = B
            cu_ptr = None
        init_ptr = None
        if initial_state is not None:
            init = np.ascontiguousarray(initial_state, dtype=np.float32)
            if init.shape != (n_seq, H, dk, dv):
                raise ValueError(f"initial_state must be {(n_seq, H, dk, dv)}")
            init_ptr = init.ctypes.data
        o = np.zeros((B, T, H, dv))
        fs = np.zeros((n_seq, H, dk, dv))
        ptr = lambda x: None if x is None else x.ctypes.data
        rc = self._lib.oracle_recurrent_gated_fwd(
            B, T, H, Hkv, dk, dv, dt, q.ctypes.data, k.ctypes.data, v.ctypes.data,
            *(ptr(x) for x in gates), ptr(gg), float(scale), init_ptr, int(bool(reverse)), cu_ptr,
            n_seq, o.ctypes.data, fs.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return (o[0] if squeeze else o), fs

    # -- backward ----------------------------------------------------------------
    def recurrent_bwd(self, q, k, v, g_gamma, scale, d_o, d_final=None, initial_state=None,
                      reverse=False, cu_seqlens=None, want_d_init=True):
        """fp64 gradients of the forward recurrence.

        Returns (dq [.., T, H, dk], dk [.., T, Hkv, dk], dv [.., T, Hkv, dv],
        d_initial_state [N_seq, H, dk, dv] or None).  ``d_o`` has the dtype of q, k, v
        (float32 values or bf16 words); ``d_final`` is taken as float32.  Rows outside
        every packed sequence are zero.
        """
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        squeeze = q.ndim == 3
        if squeeze:
            q, k, v = q[None], k[None], v[None]
            d_o = np.asarray(d_o)[None]
        if not (q.dtype == k.dtype == v.dtype):
            raise TypeError("q, k, v must share one dtype")
        dt = _in_dtype(q)
        B, T, H, dk = q.shape
        Hkv = k.shape[2]
        dv = v.shape[3]
        if k.shape != (B, T, Hkv, dk) or v.shape != (B, T, Hkv, dv):
            raise ValueError("inconsistent q/k/v shapes")
        do_ = np.ascontiguousarray(d_o)
        if do_.dtype != q.dtype:
            raise TypeError("d_o must have the dtype of q, k, v")
        if do_.shape != (B, T, H, dv):
            raise ValueError("d_o must have the shape of o")
        g = np.ascontiguousarray(g_gamma, dtype=np.float32)
        if cu_seqlens is not None:
            cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
            n_seq = cu.shape[0] - 1
            cu_ptr = cu.ctypes.data
        else:
            n_seq = B
            cu_ptr = None
        st_shape = (n_seq, H, dk, dv)
        init_ptr = fin_ptr = None
        if initial_state is not None:
            init = np.ascontiguousarray(initial_state, dtype=np.float32)
            if init.shape != st_shape:
                raise ValueError(f"initial_state must be {st_shape}")
            init_ptr = init.ctypes.data
        if d_final is not None:
            fin = np.ascontiguousarray(d_final, dtype=np.float32)
            if fin.shape != st_shape:
                raise ValueError(f"d_final must be {st_shape}")
            fin_ptr = fin.ctypes.data
        dq = np.zeros((B, T, H, dk))
        dk_ = np.zeros((B, T, Hkv, dk))
        dv_ = np.zeros((B, T, Hkv, dv))
        d_init = np.zeros(st_shape) if want_d_init else None
        rc = self._lib.oracle_recurrent_bwd(
            B, T, H, Hkv, dk, dv, dt, q.ctypes.data, k.ctypes.data, v.ctypes.data,
            g.ctypes.data, float(scale), init_ptr, int(bool(reverse)), cu_ptr, n_seq,
            do_.ctypes.data, fin_ptr, dq.ctypes.data, dk_.ctypes.data, dv_.ctypes.data,
            d_init.ctypes.data if want_d_init else None)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        if squeeze:
            dq, dk_, dv_ = dq[0], dk_[0], dv_[0]
        return dq, dk_, dv_, d_init

    def lightning_attn(self, q, k, v, layer_idx, num_layers, softmax_scale=None,
                       initial_state=None, reverse=False, cu_seqlens=None):
        """The lightning_attn wrapper: default scale dk^-1/2 and the layer decay."""
        if softmax_scale is None:
            softmax_scale = float(np.float32(k.shape[-1] ** -0.5))
        g = self.lightning_g_gamma(q.shape[-2], layer_idx, num_layers)
        return self.recurrent_fwd(q, k, v, g, softmax_scale, initial_state, reverse, cu_seqlens)


_default: Oracle | None = None


def load(path: str | None = None) -> Oracle:
    """Load (building first if needed) the oracle library."""
    global _default
    if path is not None:
        return Oracle(path)
    if _default is None:
        if not os.path.exists(LIB):
            build()
        _default = Oracle(LIB)
    return _default

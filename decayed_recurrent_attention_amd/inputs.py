"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and rounds them to the input precision; it
holds none of the attention method's arithmetic (no decay schedule, no
recurrence).  Both the GPU path and the CPU oracle receive exactly the arrays
it returns.

Recipe (stated once here and in the design notes):

* Every random tensor is drawn in flattened C order, in blocks of ``BLOCK``
  elements; block ``i`` of stream ``s`` comes from
  ``numpy.random.Generator(PCG64(SeedSequence([seed, s, i])))``.  The result is
  therefore independent of how many threads draw it.
* Streams: 0 = q, 1 = k, 2 = v, 3 = initial_state, 4 = sequence lengths.
* q, k, v are standard normal float32, then rounded to bf16 (round to nearest
  even) for bf16 workloads; fp32 workloads keep the float32 values.
* initial_state (when used) is normal with standard deviation 0.1, float32.
* Packed lengths are uniform integers in [lo, hi] (both ends included).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK = 1 << 22

STREAM_Q, STREAM_K, STREAM_V, STREAM_INIT, STREAM_LENS = 0, 1, 2, 3, 4
STREAM_DO, STREAM_DFINAL = 5, 6  # gradients for the backward
STREAM_G, STREAM_GK, STREAM_GV = 7, 8, 9  # log-decay gates of the gated recurrence


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_words(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16 words."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_values(words: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 words."""
    return (np.asarray(words, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_block(seed: int, stream: int, i: int, n: int, std: float, as_bf16: bool):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, i])))
    x = rng.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_words(x) if as_bf16 else x


def normal(shape, seed: int, stream: int, std: float = 1.0, as_bf16: bool = False) -> np.ndarray:
    """Seeded normal tensor (float32, or bf16 words when ``as_bf16``)."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16 if as_bf16 else np.float32)
    nblk = (total + BLOCK - 1) // BLOCK

    def fill(i):
        lo = i * BLOCK
        hi = min(total, lo + BLOCK)
        out[lo:hi] = _normal_block(seed, stream, i, hi - lo, std, as_bf16)

    if nblk <= 1:
        for i in range(nblk):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Seeded sequence lengths, uniform in [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, STREAM_LENS, 0])))
    return rng.integers(lo, hi, endpoint=True, size=n).astype(np.int64)


@dataclass
class Workload:
    """One synthetic problem: shapes, dtype and the arguments of lightning_attn."""

    name: str
    batch: int
    seqlen: int  # tokens per batch row; total packed tokens when varlen
    num_heads: int
    num_kv_heads: int
    dk: int
    dv: int
    dtype: str  # "bf16" or "f32"
    layer_idx: int
    num_layers: int
    reverse: bool = False
    seq_lens: list | None = None  # packed varlen lengths (batch must be 1)
    init_std: float | None = None  # initial_state ~ N(0, init_std) when set
    seed: int = 0
    scale: float = field(default=0.0)

    def __post_init__(self):
        if not self.scale:
            self.scale = float(np.float32(1.0 / np.sqrt(self.dk)))

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens) if self.seq_lens is not None else self.batch

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def cu_seqlens(self) -> np.ndarray | None:
        if self.seq_lens is None:
            return None
        return np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int64)

    def make(self) -> dict:
        """Draw q, k, v (and initial_state) for this workload."""
        bf = self.dtype == "bf16"
        B, T, H, Hkv = self.batch, self.seqlen, self.num_heads, self.num_kv_heads
        out = {
            "q": normal((B, T, H, self.dk), self.seed, STREAM_Q, as_bf16=bf),
            "k": normal((B, T, Hkv, self.dk), self.seed, STREAM_K, as_bf16=bf),
            "v": normal((B, T, Hkv, self.dv), self.seed, STREAM_V, as_bf16=bf),
            "cu_seqlens": self.cu_seqlens(),
            "initial_state": None,
        }
        if self.init_std is not None:
            out["initial_state"] = normal((self.num_seqs, H, self.dk, self.dv), self.seed,
                                          STREAM_INIT, std=self.init_std)
        return out

    def make_gates(self, which=("g",), gmax: float = 0.5) -> dict:
        """Draw log-decay gates, uniform in [-gmax, 0), in the input dtype: g and gk are
        [B, T, H, dk], gv is [B, T, H, dv]; gates not named are None."""
        B, T, H = self.batch, self.seqlen, self.num_heads
        out = {}
        for name, d, stream in (("g", self.dk, STREAM_G), ("gk", self.dk, STREAM_GK), ("gv", self.dv, STREAM_GV)):
            if name not in which:
                out[name] = None
                continue
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([self.seed, stream, 0])))
            x = (-gmax * rng.random((B, T, H, d), dtype=np.float32)).astype(np.float32)
            out[name] = bf16_words(x) if self.dtype == "bf16" else x
        return out

    def make_grads(self, final_std: float | None = 1.0) -> dict:
        """Draw an output gradient d_o (the shape of o, in the input dtype like q, k, v)
        and, unless ``final_std`` is None, a float32 final-state gradient d_final_state."""
        B, T, H = self.batch, self.seqlen, self.num_heads
        bf = self.dtype == "bf16"
        out = {"d_o": normal((B, T, H, self.dv), self.seed, STREAM_DO, as_bf16=bf), "d_final_state": None}
        if final_std is not None:
            out["d_final_state"] = normal((self.num_seqs, H, self.dk, self.dv), self.seed,
                                          STREAM_DFINAL, std=final_std)
        return out


def tiny_fp32(seqlen: int = 256) -> Workload:
    """fp32, B=1, H=2, d=16, layer 5 of 12."""
    return Workload("tiny_fp32_b1_h2_d16", 1, seqlen, 2, 2, 16, 16, "f32", 5, 12)


def bf16_d64(seqlen: int = 2048) -> Workload:
    """bf16, B=2, H=Hkv=8, d=64, layer 5 of 12."""
    return Workload("bf16_b2_h8_d64", 2, seqlen, 8, 8, 64, 64, "bf16", 5, 12)


def long_d128(seqlen: int = 32768, batch: int = 4) -> Workload:
    """bf16, B=4, H=Hkv=32, d=128, layer 0 of 12 (the long-sequence sweep)."""
    return Workload(f"bf16_b{batch}_h32_d128_n{seqlen}", batch, seqlen, 32, 32, 128, 128,
                    "bf16", 0, 12)


def d192(seqlen: int = 2048) -> Workload:
    """bf16, B=2, H=12, d=192, layer 3 of 24 (non power-of-two head dim)."""
    return Workload("bf16_b2_h12_d192", 2, seqlen, 12, 12, 192, 192, "bf16", 3, 24)


def varlen_gqa(reverse: bool = False, num_seqs: int = 16, lo: int = 128, hi: int = 8192,
               seed: int = 0) -> Workload:
    """bf16 packed varlen, H=16 query / 4 kv heads, d=128, random initial state."""
    lens = lengths(num_seqs, lo, hi, seed)
    return Workload(f"bf16_varlen{num_seqs}_h16_kv4_d128" + ("_rev" if reverse else ""), 1,
                    int(lens.sum()), 16, 4, 128, 128, "bf16", 6, 12, reverse=reverse,
                    seq_lens=[int(x) for x in lens], init_std=0.1, seed=seed)


SWEEP_N = (512, 1024, 2048, 4096, 8192, 16384, 32768)

"""Seeded synthetic inputs for the top-K KL distillation loss.

This module is shared by the CPU oracle and the GPU library's tests and bench.
It holds no arithmetic of the loss itself: it only draws random numbers and
rounds them to the storage formats the GPU path consumes.

Workload recipe (the pages train on real corpora; these draws stand in for
them with the same shapes):
  * hidden[S, H] ~ N(0, 1) and W[V, H] ~ N(0, 1/H), drawn in fp32 and rounded
    to bf16 with round-to-nearest-even (kept fp32 for the fp32 case);
  * teacher cache (per position the K most likely ids with their logits, as
    "Making Knowledge Distillation Cheap Enough to Run at Scale", section
    "offline top-K logits", describes a top-100 cache): K distinct ids drawn
    uniformly from [0, V); logits 8 - 1.5*ln(k+1) + N(0, variance 0.5) for
    k = 0..K-1, each row sorted descending, stored bf16 (or fp32);
  * generator: numpy PCG64 with the caller's seed.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "draw_distinct_ids",
    "make_problem",
    "Problem",
]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    NaN is kept NaN (quiet); infinities stay infinities.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> 16
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, (u >> 16) | np.uint32(0x40), rounded)
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw_distinct_ids(rng: np.random.Generator, S: int, K: int, V: int) -> np.ndarray:
    """S rows of K distinct ids, uniform over [0, V); int32 [S, K].

    Rows are drawn with replacement and the rows that collide are redrawn until
    none does; for dense cases (K > V/4) each row is a random K-subset.
    """
    if K > V:
        raise ValueError("K must not exceed V")
    if S == 0:
        return np.zeros((0, K), dtype=np.int32)
    if 4 * K > V:
        out = np.empty((S, K), dtype=np.int64)
        for t in range(S):
            out[t] = rng.choice(V, size=K, replace=False)
        return out.astype(np.int32)
    ids = rng.integers(0, V, size=(S, K), dtype=np.int64)
    while True:
        srt = np.sort(ids, axis=1)
        bad = np.nonzero((srt[:, 1:] == srt[:, :-1]).any(axis=1))[0]
        if bad.size == 0:
            break
        ids[bad] = rng.integers(0, V, size=(bad.size, K), dtype=np.int64)
    return ids.astype(np.int32)


class Problem:
    """One synthetic instance. Arrays are host numpy arrays.

    hidden / W / topk_logits are held in their storage format:
      * dtype "bf16": uint16 bit patterns (``*_bits``) plus the exact fp32 widening;
      * dtype "f32": fp32 values (``*_bits`` is None).
    """

    def __init__(self, S, H, V, K, T, chunk, hw_dtype, tl_dtype, hidden, W, ids,
                 tlogits, hidden_bits=None, W_bits=None, tl_bits=None):
        self.S, self.H, self.V, self.K = S, H, V, K
        self.T, self.chunk = T, chunk
        self.hw_dtype, self.tl_dtype = hw_dtype, tl_dtype
        self.hidden, self.W, self.ids, self.tlogits = hidden, W, ids, tlogits
        self.hidden_bits, self.W_bits, self.tl_bits = hidden_bits, W_bits, tl_bits

    def hidden_storage(self):
        return self.hidden_bits if self.hw_dtype == "bf16" else self.hidden

    def W_storage(self):
        return self.W_bits if self.hw_dtype == "bf16" else self.W

    def tl_storage(self):
        return self.tl_bits if self.tl_dtype == "bf16" else self.tlogits


def make_problem(S: int, H: int, V: int, K: int, *, T: float = 1.0, chunk: int = 1024,
                 hw_dtype: str = "bf16", tl_dtype: str = "bf16", seed: int = 0,
                 hidden_std: float = 1.0, w_std: float | None = None) -> Problem:
    """Draw one instance of the workload recipe described in the module docstring."""
    if hw_dtype not in ("bf16", "f32") or tl_dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    rng = np.random.Generator(np.random.PCG64(seed))
    if w_std is None:
        w_std = 1.0 / np.sqrt(H)
    hidden = rng.standard_normal((S, H), dtype=np.float32)
    if hidden_std != 1.0:
        hidden *= np.float32(hidden_std)
    W = rng.standard_normal((V, H), dtype=np.float32)
    W *= np.float32(w_std)
    ids = draw_distinct_ids(rng, S, K, V)
    k = np.arange(K, dtype=np.float64)
    base = (8.0 - 1.5 * np.log(k + 1.0)).astype(np.float32)
    noise = rng.standard_normal((S, K), dtype=np.float32) * np.float32(np.sqrt(0.5))
    tl = -np.sort(-(base[None, :] + noise), axis=1)
    hb = wb = tb = None
    if hw_dtype == "bf16":
        hb = bf16_bits_from_f32(hidden)
        hidden = f32_from_bf16_bits(hb)
        wb = bf16_bits_from_f32(W)
        W = f32_from_bf16_bits(wb)
    if tl_dtype == "bf16":
        tb = bf16_bits_from_f32(tl)
        tl = f32_from_bf16_bits(tb)
    return Problem(S, H, V, K, T, chunk, hw_dtype, tl_dtype, hidden, W, ids, tl, hb, wb, tb)

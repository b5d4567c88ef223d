"""Seeded synthetic video-token workloads shared by the tests, the bench and the oracle.

This module holds the input recipe only: shapes, random streams and the cast to the
storage dtype. It contains none of the attention method's arithmetic (no pooling,
scores, softmax, selection or attention), so it can serve both the CPU oracle and the
GPU path without coupling them.

The workloads imitate the video DiT attention inputs that the pages evaluate on
(SpargeAttention2 §4: Wan2.1 1.3B at 480p and 14B at 720p; Veda §4: sequences up to
245K tokens; SALAD §4: Wan2.1-1.3B at 480p, about 30k tokens). No model weights or
video data exist here; seeded synthetic tensors of the same shapes stand in for them.

Recipe (all draws in float64, then rounded to the storage dtype):
  * tokens lie on a (T, Hg, W) grid; token n = (t*Hg + y)*W + x;
  * every random stream is numpy ``Generator(PCG64(SeedSequence(key)))`` with
    key = [seed, stream, b, h] for per-head tensors, [seed, 4, b] for sink positions and
    [seed, 5] for the blend weights;
  * Q, K, V noise ~ N(0, 1) (streams 0, 1, 2);
  * a positional term shared by Q and K of head h (stream 3):
    P[n, c] = sum_{m<8} A * sin(wt*t + wy*y + wx*x + phi), with wt, wy, wx ~ U(0, 0.1*pi)
    radians per grid step (smooth over >= 20 steps) and phi ~ U(0, 2*pi), drawn per
    (channel c, term m), and amplitude A = 1.5 for each of the 8 sinusoids. The
    amplitude and the frequency range set how peaked the pooled block scores are, so
    they set the realised sparsity; they were fixed once so that the hybrid rule lands
    near the sparsities the workloads aim at (about 90-95% for the 480p and 720p
    shapes, 97% for the sparse+linear one) and are never tuned per run;
  * Q = noise + P, K = noise + P, V = noise;
  * ``n_sinks`` token positions per batch (stream 4, without replacement) whose K rows
    are multiplied by ``sink_scale`` after P is added (attention sinks);
  * the blend weight alpha [H, D] ~ U(0.5, 1) in float32 (stream 5);
  * cast: float64 -> float32 (round to nearest even) -> bfloat16 (round to nearest
    even) when the dtype is bf16. bf16 tensors are returned as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

N_POS_TERMS = 8
POS_AMPLITUDE = 1.5
POS_MAX_FREQ = 2.0 * math.pi * 0.05

STREAM_Q, STREAM_K, STREAM_V, STREAM_POS, STREAM_SINK, STREAM_ALPHA = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    grid: Tuple[int, int, int]  # (T, Hg, W)
    dtype: str                  # "fp32" | "bf16"
    block_q: int
    block_kv: int
    topk: float                 # fraction of KV blocks kept by the top-k rule
    top_p: float                # cumulative-mass threshold of the top-p rule
    n_sinks: int
    sink_scale: float = 8.0
    linear: bool = False        # blend in the linear-attention branch
    seed: int = 0

    @property
    def N(self) -> int:
        t, y, x = self.grid
        return t * y * x

    @property
    def n_qblk(self) -> int:
        return -(-self.N // self.block_q)

    @property
    def n_kvblk(self) -> int:
        return -(-self.N // self.block_kv)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.n_qblk

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five measured workloads.
TINY_FP32 = Workload("tiny_fp32", 1, 2, 64, (4, 16, 16), "fp32", 64, 64, 0.25, 0.90, 4)
WAN13B_480P = Workload("wan13b_480p", 1, 12, 128, (21, 30, 52), "bf16", 128, 64, 0.05, 0.90, 16)
WAN14B_720P = Workload("wan14b_720p", 1, 40, 128, (21, 45, 80), "bf16", 128, 64, 0.03, 0.85, 16)
LONG_245K = Workload("long_245k", 1, 8, 128, (60, 64, 64), "bf16", 128, 64, 0.02, 0.85, 16)
SPARSE_LINEAR = Workload("sparse_linear", 1, 12, 128, (21, 30, 52), "bf16", 128, 64, 0.02, 0.80, 16,
                         linear=True)

CONFIGS: Dict[str, Workload] = {w.name: w for w in
                                (TINY_FP32, WAN13B_480P, WAN14B_720P, LONG_245K, SPARSE_LINEAR)}


def long_sweep() -> List[Workload]:
    """The sequence-length sweep of the long workload: T in {8, 15, 30, 60} on 64x64."""
    return [LONG_245K.replace(name=f"long_T{t}", grid=(t, 64, 64)) for t in (8, 15, 30, 60)]


# the sweep points are also addressable by name (T = 60 is long_245k itself)
SWEEP: Dict[str, Workload] = {w.name: w for w in long_sweep()}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 (RNE), returned as uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def grid_coords(grid: Tuple[int, int, int]) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    T, Hg, W = grid
    n = np.arange(T * Hg * W)
    return n // (Hg * W), (n // W) % Hg, n % W


def positional_term(w: Workload, b: int, h: int) -> np.ndarray:
    """P [N, D] float64 for head h of batch b."""
    g = _rng(w.seed, STREAM_POS, b, h)
    omega = g.uniform(0.0, POS_MAX_FREQ, size=(3, w.D, N_POS_TERMS))
    phase = g.uniform(0.0, 2.0 * math.pi, size=(w.D, N_POS_TERMS))
    T, Hg, W = w.grid
    t = np.arange(T, dtype=np.float64)
    y = np.arange(Hg, dtype=np.float64)
    x = np.arange(W, dtype=np.float64)
    ang_yx = (y[:, None, None, None] * omega[1] + x[None, :, None, None] * omega[2])  # [Hg,W,D,M]
    out = np.empty((T, Hg, W, w.D), dtype=np.float64)
    for ti in range(T):
        ang = ang_yx + (t[ti] * omega[0] + phase)
        out[ti] = np.sin(ang).sum(axis=-1)
    out *= POS_AMPLITUDE
    return out.reshape(T * Hg * W, w.D)


def sink_positions(w: Workload, b: int) -> np.ndarray:
    g = _rng(w.seed, STREAM_SINK, b)
    if w.n_sinks == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(g.choice(w.N, size=min(w.n_sinks, w.N), replace=False))


def _head(w: Workload, b: int, h: int):
    N, D = w.N, w.D
    pos = positional_term(w, b, h)
    q = _rng(w.seed, STREAM_Q, b, h).standard_normal((N, D)) + pos
    k = _rng(w.seed, STREAM_K, b, h).standard_normal((N, D)) + pos
    k[sink_positions(w, b)] *= w.sink_scale
    v = _rng(w.seed, STREAM_V, b, h).standard_normal((N, D))
    if w.dtype == "bf16":
        return f64_to_bf16_bits(q), f64_to_bf16_bits(k), f64_to_bf16_bits(v)
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


def make_alpha(w: Workload) -> np.ndarray:
    return _rng(w.seed, STREAM_ALPHA).uniform(0.5, 1.0, size=(w.H, w.D)).astype(np.float32)


def make_inputs(w: Workload, heads: Optional[List[Tuple[int, int]]] = None,
                workers: Optional[int] = None):
    """Q, K, V as [B, H, N, D] arrays (uint16 bf16 bits or float32) and alpha [H, D].

    ``heads`` limits generation to some (b, h) pairs (the rest stay zero), which keeps
    sampled checks of the large workloads cheap. Heads are independent streams, so
    they are generated in parallel threads with identical results.
    """
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    shape = (w.B, w.H, w.N, w.D)
    q = np.zeros(shape, dt)
    k = np.zeros(shape, dt)
    v = np.zeros(shape, dt)
    todo = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    nw = workers or min(len(todo), max(1, min(16, os.cpu_count() or 1)))

    def job(bh):
        b, h = bh
        q[b, h], k[b, h], v[b, h] = _head(w, b, h)

    if nw <= 1:
        for bh in todo:
            job(bh)
    else:
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(job, todo))
    return q, k, v, make_alpha(w)


def to_f32(x: np.ndarray) -> np.ndarray:
    """Stored values widened exactly to float32."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else x.astype(np.float32, copy=False)


def small(name: str, B: int, H: int, N: int, D: int, dtype: str, block_q: int, block_kv: int,
          topk: float, top_p: float, n_sinks: int = 2, linear: bool = False,
          seed: int = 0) -> Workload:
    """A small test workload on a 1 x 1 x N grid (any N, so ragged tails are possible)."""
    return Workload(name, B, H, D, (1, 1, N), dtype, block_q, block_kv, topk, top_p,
                    n_sinks, linear=linear, seed=seed)

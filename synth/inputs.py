"""Seeded synthetic Q/K/V for HGA routed attention.

This module only makes inputs; it holds none of the method's arithmetic (no
summaries, scores, selection or attention). Both the CPU oracle's tests and the
GPU path read the same arrays from here.

Recipe (per workload, seed s):
  * Each (stream, b, head) slice has its own generator,
    ``default_rng(SeedSequence(s, spawn_key=(stream, b, head)))`` with streams
    Q=0, K=1, V=2, planting=3, so any slice can be regenerated alone.
  * Q, K, V entries are float32 N(0, 1).
  * RoPE (rotate-half pairing of dims i and i + D/2, inverse frequency
    theta^(-2i/D)) is applied in float64 to Q at positions T-Nq..T-1 and to K at
    positions 0..T-1. V gets no rotation. The library consumes these post-RoPE
    values, as a KV cache stores them.
  * Planting (bf16 workloads with ``plants > 0``): for every query head h, P
    distinct chunks are chosen among chunks 1 .. L0-1 (L0 = chunk of the first
    query), disjoint across the query heads that share a KV head, with
    P = min(plants, k_chunk, floor(#eligible / r)). Every key row k of a planted
    chunk is replaced by |k| * (c * qh + sqrt(1 - c^2) * e), where qh is the unit
    post-RoPE query of head h at the last position, e is a unit vector
    orthogonal to qh drawn from N(0, I), and c is the workload's cosine (0.6).
    Each planted key then has cosine exactly c with the last query.
  * Values are finally rounded to the workload dtype (round-to-nearest-even for
    bf16) and returned as float32 arrays holding exactly those values.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

from .workloads import Workload

STREAM_Q, STREAM_K, STREAM_V, STREAM_PLANT = 0, 1, 2, 3


def _rng(seed: int, stream: int, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(stream, b, h)))


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to float32 (``f32``) or to bfloat16 with ties to even (``bf16``),
    returned as a float32 array."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE in float64 on the last axis; ``positions`` indexes axis -2."""
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / d)
    ang = positions.astype(np.float64)[:, None] * inv_freq[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x = x.astype(np.float64)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def query_positions(w: Workload) -> np.ndarray:
    return np.arange(w.T - w.Nq, w.T, dtype=np.int64)


def gen_q(w: Workload, seed: int = 0) -> np.ndarray:
    """Post-RoPE queries ``[B, Hq, Nq, D]`` (float32 holding dtype values)."""
    pos = query_positions(w)
    out = np.empty((w.B, w.Hq, w.Nq, w.D), dtype=np.float32)
    for b in range(w.B):
        for h in range(w.Hq):
            raw = _rng(seed, STREAM_Q, b, h).standard_normal((w.Nq, w.D), dtype=np.float32)
            out[b, h] = round_to_dtype(rope(raw, pos, w.theta), w.dtype)
    return out


def plant_count(w: Workload) -> int:
    if w.plants <= 0:
        return 0
    n_elig = len(_eligible_chunks(w))
    return max(0, min(w.plants, w.k_chunk, n_elig // w.r))


def _eligible_chunks(w: Workload) -> np.ndarray:
    first_query_chunk = (w.T - w.Nq) // w.chunk
    return np.arange(1, first_query_chunk, dtype=np.int64)


def gen_kv_slice(w: Workload, seed: int, b: int, kvh: int, Q: np.ndarray):
    """K and V of one (sequence, KV head): ``[T, D]`` each, plus the planted
    chunks of each of its query heads ``{h: [chunk ids]}``."""
    kpos = np.arange(w.T, dtype=np.int64)
    k = rope(_rng(seed, STREAM_K, b, kvh).standard_normal((w.T, w.D), dtype=np.float32),
             kpos, w.theta)
    v = _rng(seed, STREAM_V, b, kvh).standard_normal((w.T, w.D), dtype=np.float32)
    planted: dict[int, list[int]] = {}
    P = plant_count(w)
    if P > 0:
        prng = _rng(seed, STREAM_PLANT, b, kvh)
        chosen = prng.choice(_eligible_chunks(w), size=w.r * P, replace=False)
        c = w.cosine
        s = np.sqrt(1.0 - c * c)
        for j in range(w.r):
            h = kvh * w.r + j
            qh = Q[b, h, w.Nq - 1].astype(np.float64)
            qh = qh / np.linalg.norm(qh)
            mine = sorted(int(x) for x in chosen[j * P:(j + 1) * P])
            planted[h] = mine
            for ch in mine:
                lo, hi = ch * w.chunk, min((ch + 1) * w.chunk, w.T)
                g = prng.standard_normal((hi - lo, w.D))
                g = g - (g @ qh)[:, None] * qh[None, :]
                e = g / np.linalg.norm(g, axis=1, keepdims=True)
                norms = np.linalg.norm(k[lo:hi], axis=1, keepdims=True)
                k[lo:hi] = norms * (c * qh[None, :] + s * e)
    return round_to_dtype(k, w.dtype), round_to_dtype(v, w.dtype), planted


@dataclass
class Inputs:
    workload: Workload
    seed: int
    Q: np.ndarray                      # [B, Hq, Nq, D]
    K: np.ndarray                      # [B, Hkv, T, D]
    V: np.ndarray                      # [B, Hkv, T, D]
    planted: dict = field(default_factory=dict)   # (b, h) -> sorted planted chunk ids


def generate(w: Workload, seed: int = 0, threads: int | None = None) -> Inputs:
    Q = gen_q(w, seed)
    K = np.empty((w.B, w.Hkv, w.T, w.D), dtype=np.float32)
    V = np.empty_like(K)
    planted: dict = {}

    def one(bh):
        b, kvh = bh
        k, v, pl = gen_kv_slice(w, seed, b, kvh, Q)
        K[b, kvh] = k
        V[b, kvh] = v
        return b, pl

    jobs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    n = threads or min(16, len(os.sched_getaffinity(0)), len(jobs))
    with ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        for b, pl in ex.map(one, jobs):
            for h, chunks in pl.items():
                planted[(b, h)] = chunks
    return Inputs(w, seed, Q, K, V, planted)

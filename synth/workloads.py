"""Named synthetic workloads for HGA routed attention.

Every workload is a shape plus routing hyperparameters; no values live here.
Head layout and RoPE base follow the model the HGA abstract evaluates on
(Qwen3-30B-A3B: 32 query heads, 4 KV heads, head_dim 128, RoPE base 1e6).
The routed budget follows the abstract's sparsity of roughly 3%: k_group * group
tokens out of T (3.125% at every long-context shape below).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    B: int          # sequences
    Hq: int         # query heads
    Hkv: int        # KV heads (Hq % Hkv == 0; consecutive query heads share one)
    D: int          # head dim
    T: int          # keys in the cache
    Nq: int         # queries per sequence, at positions T-Nq .. T-1
    chunk: int      # tokens per chunk (C)
    group: int      # tokens per group (G); chunk % group == 0
    k_chunk: int    # chunks kept by score, besides the forced first and last
    k_group: int    # groups kept among the candidates of the kept chunks
    theta: float    # RoPE base
    dtype: str      # "f32" or "bf16": type of Q, K, V
    plants: int     # planted q-aligned chunks per query head (0 = none)
    cosine: float = 0.6
    host_kv: bool = False   # full K/V kept in pinned host memory (only summaries in HBM)

    @property
    def r(self) -> int:
        return self.Hq // self.Hkv

    @property
    def n_chunks(self) -> int:
        return -(-self.T // self.chunk)

    @property
    def n_groups(self) -> int:
        return -(-self.T // self.group)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _decode(T: int, B: int, name: str) -> Workload:
    # Budget held at ~3% of context: k_group*32 = T/32 tokens, k_chunk = T/2048 chunks.
    return Workload(name=name, B=B, Hq=32, Hkv=4, D=128, T=T, Nq=1, chunk=256, group=32,
                    k_chunk=max(1, T // 2048), k_group=max(1, T // 1024), theta=1e6,
                    dtype="bf16", plants=8)


TINY = Workload(name="tiny-f32-t1024-nq16", B=1, Hq=1, Hkv=1, D=64, T=1024, Nq=16,
                chunk=64, group=16, k_chunk=4, k_group=4, theta=1e4, dtype="f32", plants=0)
# Same inputs with every chunk and group kept: must reproduce dense causal attention.
TINY_ALL = TINY.with_(name="tiny-f32-t1024-nq16-all", k_chunk=16, k_group=64)

DECODE_64K = _decode(65536, 1, "qwen3-30b-a3b-decode-b1-t65536")
SWEEP = {T: _decode(T, 16, f"qwen3-30b-a3b-decode-b16-t{T}")
         for T in (4096, 8192, 16384, 32768, 65536)}
PREFILL = Workload(name="qwen3-30b-a3b-prefill-nq4096-t65536", B=1, Hq=32, Hkv=4, D=128,
                   T=65536, Nq=4096, chunk=256, group=32, k_chunk=32, k_group=64,
                   theta=1e6, dtype="bf16", plants=8)
HOST_TIER = _decode(262144, 4, "qwen3-30b-a3b-host-tier-b4-t262144").with_(host_kv=True)

ALL = {w.name: w for w in [TINY, TINY_ALL, DECODE_64K, *SWEEP.values(), PREFILL, HOST_TIER]}

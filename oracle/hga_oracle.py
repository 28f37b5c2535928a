"""Plain CPU oracle for Hierarchical Global Attention (HGA) routed attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the HIP
library and its Python binding) never calls it, and it shares no code, table or
helper with that path.

Source: the abstract of "Hierarchical Global Attention (HGA)", arXiv 2606.30709,
as shown on its searcharxiv.com page (cited below as [HGA abstract]). It
describes the method in three steps: score compact RoPE-aware chunk summaries and
retrieve the relevant chunks; inside those chunks, route only the most relevant
groups; then run exact token-level attention over the retrieved tokens, as a
drop-in for dense causal attention with the model's projections unchanged.

Every step is written in float64 NumPy, one query at a time, in the order the
method states. Readings where the abstract is silent (each listed in the design
notes of this repository):
  * summary = arithmetic mean of the post-RoPE keys of a group or chunk
    (mean over the keys present for a short last group/chunk);
  * score = q . summary / sqrt(D), the logit of the mean key;
  * the first chunk and the query's own chunk are always kept, in addition to
    the k_chunk best chunks among the others;
  * groups of the forced chunks compete in the group selection like all others;
  * group selection is global over all candidate groups of the kept chunks;
  * a chunk or group is a candidate iff its first position is <= p;
  * ties go to the lower index; index lists are ascending and -1 padded;
  * query i of Nq sits at position p = T - Nq + i and attends to j <= p;
  * softmax scale 1/sqrt(D) unless given.

Parity pins: every function here is pinned by tests that do not reuse its code
(closed forms, brute force over subsets, torch's CPU attention on the gathered
tokens, a hand-worked example, invariants of the input generator).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# --------------------------------------------------------------------------
# Step 1 of [HGA abstract]: compact summaries of the keys.
# --------------------------------------------------------------------------
def build_summaries(K, chunk: int, group: int):
    """Mean post-RoPE key of every chunk and every group.

    K: [B, Hkv, T, D]. Returns (chunk_mean [B, Hkv, n_c, D],
    group_mean [B, Hkv, n_g, D]) in float64, n_c = ceil(T/chunk),
    n_g = ceil(T/group).
    """
    K = np.asarray(K, dtype=np.float64)
    T = K.shape[2]
    n_c = -(-T // chunk)
    n_g = -(-T // group)
    chunk_mean = np.stack([K[:, :, c * chunk:min((c + 1) * chunk, T)].mean(axis=2)
                           for c in range(n_c)], axis=2)
    group_mean = np.stack([K[:, :, g * group:min((g + 1) * group, T)].mean(axis=2)
                           for g in range(n_g)], axis=2)
    return chunk_mean, group_mean


# --------------------------------------------------------------------------
# Selection helper: the k best items by (score descending, index ascending).
# --------------------------------------------------------------------------
def top_k(ids, scores, k: int):
    """Returns (kept ids ascending, gap) where gap is the k-th best score minus
    the (k+1)-th best (inf if nothing is dropped)."""
    ids = [int(i) for i in ids]
    scores = [float(s) for s in scores]
    order = sorted(range(len(ids)), key=lambda t: (-scores[t], ids[t]))
    if len(ids) <= k:
        return sorted(ids), math.inf
    kept = sorted(ids[t] for t in order[:k])
    gap = scores[order[k - 1]] - scores[order[k]] if k > 0 else math.inf
    return kept, gap


def score(q, summary_rows, scale: float | None = None):
    """Score of each summary row for query q: q . row * scale (scale 1/sqrt(D) by default)."""
    q = np.asarray(q, dtype=np.float64)
    scale = 1.0 / math.sqrt(q.shape[0]) if scale is None else scale
    return (np.asarray(summary_rows, dtype=np.float64) @ q) * scale


@dataclass
class QueryRoute:
    chunks: list          # kept chunk ids, ascending
    groups: list          # kept group ids, ascending
    chunk_scores: np.ndarray   # score of chunks 0..L
    candidates: list      # candidate group ids, ascending
    cand_scores: np.ndarray
    chunk_gap: float      # k-th vs (k+1)-th among the chunks that compete (inf if none dropped)
    group_gap: float


# --------------------------------------------------------------------------
# Steps 1-2 of [HGA abstract] for one query: chunk retrieval, group refinement.
# --------------------------------------------------------------------------
def route_query(q, chunk_mean_h, group_mean_h, p: int, chunk: int, group: int,
                k_chunk: int, k_group: int, scale: float | None = None) -> QueryRoute:
    n_g = group_mean_h.shape[0]
    L = p // chunk                                     # the query's own chunk
    chunk_scores = score(q, chunk_mean_h[:L + 1], scale)
    if L + 1 <= k_chunk + 2:
        chunks, chunk_gap = list(range(L + 1)), math.inf
    else:
        middle = list(range(1, L))
        best, chunk_gap = top_k(middle, chunk_scores[1:L], k_chunk)
        chunks = sorted({0, L, *best})
    per_chunk = chunk // group
    candidates = [g for c in chunks for g in range(c * per_chunk, (c + 1) * per_chunk)
                  if g < n_g and g * group <= p]
    cand_scores = score(q, np.asarray(group_mean_h)[candidates], scale)
    groups, group_gap = top_k(candidates, cand_scores, k_group)
    return QueryRoute(chunks, groups, chunk_scores, candidates, cand_scores,
                      chunk_gap, group_gap)


def route(Q, chunk_mean, group_mean, T: int, chunk: int, group: int, k_chunk: int,
          k_group: int, scale: float | None = None):
    """Routes every query. Q: [B, Hq, Nq, D]; summaries [B, Hkv, n, D].

    Returns (chunk_idx [B,Hq,Nq,k_chunk+2], group_idx [B,Hq,Nq,k_group]) as int32,
    ascending and -1 padded, plus the per-query QueryRoute records."""
    Q = np.asarray(Q, dtype=np.float64)
    B, Hq, Nq, _ = Q.shape
    r = Hq // chunk_mean.shape[1]
    chunk_idx = np.full((B, Hq, Nq, k_chunk + 2), -1, dtype=np.int32)
    group_idx = np.full((B, Hq, Nq, k_group), -1, dtype=np.int32)
    records = {}
    for b in range(B):
        for h in range(Hq):
            kv = h // r
            for i in range(Nq):
                rq = route_query(Q[b, h, i], chunk_mean[b, kv], group_mean[b, kv], T - Nq + i,
                                 chunk, group, k_chunk, k_group, scale)
                chunk_idx[b, h, i, :len(rq.chunks)] = rq.chunks
                group_idx[b, h, i, :len(rq.groups)] = rq.groups
                records[(b, h, i)] = rq
    return chunk_idx, group_idx, records


# --------------------------------------------------------------------------
# Step 3 of [HGA abstract]: exact token attention over the routed tokens.
# --------------------------------------------------------------------------
def routed_tokens(group_ids, group: int, p: int, T: int):
    """Token positions of the listed groups (-1 entries ignored) that are <= p."""
    toks = set()
    for g in group_ids:
        g = int(g)
        if g < 0:
            continue
        toks.update(j for j in range(g * group, min((g + 1) * group, T)) if j <= p)
    return sorted(toks)


def attend_tokens(q, K_h, V_h, tokens, scale: float | None = None):
    """Softmax attention of one query over the given token positions.
    Returns (output [D], log-sum-exp of the scaled logits)."""
    q = np.asarray(q, dtype=np.float64)
    scale = 1.0 / math.sqrt(q.shape[0]) if scale is None else scale
    k = np.asarray(K_h[tokens], dtype=np.float64)
    v = np.asarray(V_h[tokens], dtype=np.float64)
    logits = (k @ q) * scale
    m = logits.max()
    w = np.exp(logits - m)
    s = w.sum()
    return (w @ v) / s, m + math.log(s)


def attend(Q, K, V, group_idx, group: int, scale: float | None = None):
    """Exact attention of every query over its routed tokens.
    Q [B,Hq,Nq,D], K/V [B,Hkv,T,D], group_idx [B,Hq,Nq,k]. Returns (O, lse)."""
    Q = np.asarray(Q, dtype=np.float64)
    B, Hq, Nq, D = Q.shape
    Hkv, T = K.shape[1], K.shape[2]
    r = Hq // Hkv
    O = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            for i in range(Nq):
                p = T - Nq + i
                toks = routed_tokens(group_idx[b, h, i], group, p, T)
                O[b, h, i], lse[b, h, i] = attend_tokens(Q[b, h, i], K[b, h // r], V[b, h // r],
                                                         toks, scale)
    return O, lse


def dense_causal(Q, K, V, scale: float | None = None):
    """Dense causal attention: query i attends to every position j <= T - Nq + i."""
    Q = np.asarray(Q, dtype=np.float64)
    B, Hq, Nq, D = Q.shape
    Hkv, T = K.shape[1], K.shape[2]
    r = Hq // Hkv
    O = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            for i in range(Nq):
                toks = list(range(T - Nq + i + 1))
                O[b, h, i], lse[b, h, i] = attend_tokens(Q[b, h, i], K[b, h // r], V[b, h // r],
                                                         toks, scale)
    return O, lse

"""Comparison of the HIP path with the CPU oracle, shared by the GPU tests,
the smoke check and the benchmark's parity line.

Rules (tolerances stated for this method's bf16 workloads: exact routed sets
wherever the oracle's k-th vs (k+1)-th score gap exceeds 1e-3; outputs within
max-abs 2e-2 and relative 1e-2 for bf16 inputs with fp32 accumulation):
  * routed sets: equal to the oracle's wherever its gap exceeds MARGIN (chunk
    level; group level when both gaps do). For every query, whatever the gap,
    the GPU's choice is epsilon-valid: forced chunks present, right count, and
    no dropped candidate beats a kept one by more than MARGIN on the oracle's
    fp64 scores (group candidates taken from the GPU's own chunk set);
  * outputs: the GPU's O matches the oracle's attention over the GPU's own
    routed groups for every query; lse within LSE_TOL;
  * fp32 inputs: max-abs 1e-4 and relative-L2 1e-5 (fp32 accumulation over at
    most a few thousand terms of unit size).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle

MARGIN = 1e-3
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-5)}
LSE_TOL = 1e-3


@dataclass
class RouteStats:
    queries: int = 0
    chunk_exempt: int = 0
    group_exempt: int = 0
    failures: list = field(default_factory=list)

    def ok(self):
        return not self.failures


def check_summaries(cm_gpu, gm_gpu, cm_ref, gm_ref):
    for name, a, b in (("chunk", cm_gpu, cm_ref), ("group", gm_gpu, gm_ref)):
        err = np.abs(a.astype(np.float64) - b).max()
        bound = 2e-6 * max(1.0, np.abs(b).max())
        assert err <= bound, f"{name} summaries: max err {err:.3g} > {bound:.3g}"


def check_routes(Q, cm_ref, gm_ref, T, chunk, group, k_chunk, k_group, chunk_idx, group_idx,
                 records, scale=None, b_list=None, rows=None) -> RouteStats:
    """Q [B,Hq,Nq,D] (oracle dtype values); chunk_idx/group_idx from the GPU for the
    same B; cm_ref/gm_ref the oracle's summaries for the sequences in b_list.
    `rows`, if given, restricts the check to those (b, h, i) query rows."""
    B, Hq, Nq, _ = Q.shape
    Hkv = cm_ref.shape[1]
    r = Hq // Hkv
    gpc = chunk // group
    n_g = gm_ref.shape[2]
    st = RouteStats()
    b_list = list(range(B)) if b_list is None else b_list
    if rows is None:
        rows = [(b, h, i) for b in b_list for h in range(Hq) for i in range(Nq)]
    b_pos = {b: bi for bi, b in enumerate(b_list)}
    for (b, h, i) in rows:
        bi = b_pos[b]
        st.queries += 1
        rq = records[(b, h, i)]
        p = T - Nq + i
        L = p // chunk
        q = Q[b, h, i]
        gc = [int(c) for c in chunk_idx[b, h, i] if c >= 0] if chunk_idx is not None else None
        gg = [int(g) for g in group_idx[b, h, i] if g >= 0]
        tag = (b, h, i)
        # -- chunk level
        if gc is not None:
            if rq.chunk_gap > MARGIN:
                if gc != rq.chunks:
                    st.failures.append((tag, "chunk set", gc, rq.chunks))
            else:
                st.chunk_exempt += 1
            want_n = min(L + 1, k_chunk + 2)
            if len(gc) != want_n or gc != sorted(set(gc)) or gc[0] != 0 or gc[-1] != L:
                st.failures.append((tag, "chunk shape/forced", gc))
            else:
                mid_kept = [c for c in gc if 0 < c < L]
                mid_drop = [c for c in range(1, L) if c not in set(gc)]
                if mid_kept and mid_drop:
                    s = rq.chunk_scores
                    if min(s[c] for c in mid_kept) < max(s[c] for c in mid_drop) - MARGIN:
                        st.failures.append((tag, "chunk not eps-valid"))
        else:
            gc = rq.chunks
        # -- group level
        exact = rq.chunk_gap > MARGIN and rq.group_gap > MARGIN
        if exact:
            if gg != rq.groups:
                st.failures.append((tag, "group set", gg, rq.groups))
        else:
            st.group_exempt += 1
        cands = [g for c in gc for g in range(c * gpc, (c + 1) * gpc)
                 if g < n_g and g * group <= p]
        if len(gg) != min(k_group, len(cands)) or gg != sorted(set(gg)) \
                or not set(gg) <= set(cands):
            st.failures.append((tag, "group shape/candidates", gg))
            continue
        drop = [g for g in cands if g not in set(gg)]
        if gg and drop:
            sc = oracle.score(q, gm_ref[bi, h // r][gg + drop], scale)
            if sc[:len(gg)].min() < sc[len(gg):].max() - MARGIN:
                st.failures.append((tag, "group not eps-valid"))
    return st


def check_outputs(O_gpu, lse_gpu, O_ref, lse_ref, dtype: str):
    atol, rtol = TOL[dtype]
    d = O_gpu.astype(np.float64) - O_ref
    max_abs = float(np.abs(d).max())
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(O_ref), 1e-30))
    assert max_abs <= atol, f"O max-abs {max_abs:.3g} > {atol}"
    assert rel <= rtol, f"O rel-L2 {rel:.3g} > {rtol}"
    if lse_gpu is not None:
        le = float(np.abs(lse_gpu.astype(np.float64) - lse_ref).max())
        assert le <= LSE_TOL, f"lse max err {le:.3g}"
    return max_abs, rel

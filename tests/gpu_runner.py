"""Runs the HIP path on generated inputs and the oracle beside it (test helper)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import hierarchical_sparse_attention_summaries_amd as hga
import oracle
from tests import parity

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str, device="cuda"):
    return torch.from_numpy(x).to(device=device, dtype=TORCH_DTYPE[dtype])


def to_pinned(x: np.ndarray, dtype: str):
    return torch.from_numpy(x).to(dtype=TORCH_DTYPE[dtype]).pin_memory()


def run_hip(w, inp, device="cuda", scale=0.0):
    """Summaries, routing and attention on the GPU. With w.host_kv, K and V stay
    in pinned host memory and the kernels read the routed groups from there."""
    Q = to_dev(inp.Q, w.dtype, device)
    if w.host_kv:
        K = to_pinned(inp.K, w.dtype)
        V = to_pinned(inp.V, w.dtype)
    else:
        K = to_dev(inp.K, w.dtype, device)
        V = to_dev(inp.V, w.dtype, device)
    cm, gm = hga.build_summaries(K, w.chunk, w.group)
    cidx, gidx = hga.route(Q, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group, scale=scale)
    O, lse = hga.attend(Q, K, V, gidx, w.group, scale=scale)
    torch.cuda.synchronize()
    return dict(Q=Q, K=K, V=V, cm=cm, gm=gm, cidx=cidx, gidx=gidx, O=O, lse=lse)


def np_of(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def check_workload(w, inp, out, b_list=None, scale=None):
    """Full parity of one run against the oracle on the sequences in b_list."""
    t0 = time.time()
    B = w.B
    b_list = list(range(B)) if b_list is None else b_list
    Ksub = inp.K[b_list]
    cm_ref, gm_ref = oracle.build_summaries(Ksub, w.chunk, w.group)
    parity.check_summaries(np_of(out["cm"])[b_list], np_of(out["gm"])[b_list], cm_ref, gm_ref)
    Qsub = inp.Q[b_list]
    _, _, rec_sub = oracle.route(Qsub, cm_ref, gm_ref, w.T, w.chunk, w.group, w.k_chunk,
                                 w.k_group, scale)
    records = {(b_list[bi], h, i): v for (bi, h, i), v in rec_sub.items()}
    cidx = out["cidx"].cpu().numpy()
    gidx = out["gidx"].cpu().numpy()
    st = parity.check_routes(inp.Q, cm_ref, gm_ref, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                             cidx, gidx, records, scale=scale, b_list=b_list)
    assert st.ok(), st.failures[:5]
    # the oracle's attention over the GPU's own routed groups, for every query
    O_ref, lse_ref = oracle.attend(Qsub, Ksub, inp.V[b_list], gidx[b_list], w.group, scale)
    err = parity.check_outputs(np_of(out["O"])[b_list], np_of(out["lse"])[b_list], O_ref,
                               lse_ref, w.dtype)
    log(f"  parity {w.name}: queries={st.queries} chunk_exempt={st.chunk_exempt} "
        f"group_exempt={st.group_exempt} O max-abs={err[0]:.3g} rel={err[1]:.3g} "
        f"({time.time() - t0:.1f}s)")
    return st, err


def check_sampled(w, inp, out, n_rows=256, seed=1, scale=None):
    """Parity on a seeded sample of query rows (for workloads whose full oracle
    run would take minutes): summaries of every KV head, then routing and
    attention of the sampled rows, by the same rules as check_workload."""
    t0 = time.time()
    rng = np.random.default_rng(seed)
    all_rows = w.B * w.Hq * w.Nq
    pick = sorted(rng.choice(all_rows, size=min(n_rows, all_rows), replace=False).tolist())
    rows = [(x // (w.Hq * w.Nq), (x // w.Nq) % w.Hq, x % w.Nq) for x in pick]
    # Always include the last query of every head of sequence 0 (the planted one).
    rows = sorted(set(rows) | {(0, h, w.Nq - 1) for h in range(w.Hq)})
    b_list = sorted({b for b, _, _ in rows})
    cm_ref, gm_ref = oracle.build_summaries(inp.K[b_list], w.chunk, w.group)
    parity.check_summaries(np_of(out["cm"])[b_list], np_of(out["gm"])[b_list], cm_ref, gm_ref)
    r = w.Hq // w.Hkv
    bpos = {b: k for k, b in enumerate(b_list)}
    records = {}
    for (b, h, i) in rows:
        records[(b, h, i)] = oracle.route_query(inp.Q[b, h, i], cm_ref[bpos[b], h // r],
                                                gm_ref[bpos[b], h // r], w.T - w.Nq + i, w.chunk,
                                                w.group, w.k_chunk, w.k_group, scale)
    cidx = out["cidx"].cpu().numpy()
    gidx = out["gidx"].cpu().numpy()
    st = parity.check_routes(inp.Q, cm_ref, gm_ref, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                             cidx, gidx, records, scale=scale, b_list=b_list, rows=rows)
    assert st.ok(), st.failures[:5]
    O = np_of(out["O"])
    lse = np_of(out["lse"])
    O_ref = np.zeros((len(rows), w.D))
    lse_ref = np.zeros(len(rows))
    for k, (b, h, i) in enumerate(rows):
        toks = oracle.routed_tokens(gidx[b, h, i], w.group, w.T - w.Nq + i, w.T)
        O_ref[k], lse_ref[k] = oracle.attend_tokens(inp.Q[b, h, i], inp.K[b, h // r],
                                                    inp.V[b, h // r], toks, scale)
    sel = tuple(np.array(rows).T)
    err = parity.check_outputs(O[sel], lse[sel], O_ref, lse_ref, w.dtype)
    log(f"  sampled parity {w.name}: rows={st.queries} chunk_exempt={st.chunk_exempt} "
        f"group_exempt={st.group_exempt} O max-abs={err[0]:.3g} rel={err[1]:.3g} "
        f"({time.time() - t0:.1f}s)")
    return st, err


def check_ragged(w, inp, seq_lens, out):
    """Parity of a ragged batch: sequence b holds seq_lens[b] keys (a prefix of
    the generated capacity-T cache) and its queries sit at seq_lens[b]-Nq+i. The
    oracle runs on each sequence alone, on its own prefix."""
    from synth.inputs import Inputs
    results = []
    for b, Tb in enumerate(seq_lens):
        wb = w.with_(B=1, T=int(Tb))
        sub = Inputs(wb, inp.seed, inp.Q[b:b + 1], inp.K[b:b + 1, :, :Tb], inp.V[b:b + 1, :, :Tb])
        n_c, n_g = wb.n_chunks, wb.n_groups
        ob = dict(cm=out["cm"][b:b + 1, :, :n_c], gm=out["gm"][b:b + 1, :, :n_g],
                  cidx=out["cidx"][b:b + 1], gidx=out["gidx"][b:b + 1],
                  O=out["O"][b:b + 1], lse=out["lse"][b:b + 1])
        results.append(check_workload(wb, sub, ob))
    return results

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


def run_hip(w, inp, device="cuda", scale=0.0):
    Q = to_dev(inp.Q, w.dtype, device)
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

"""Seeded random small shapes through every routing path, against the oracle.

Each case draws batch, heads (GQA ratio 1..8), head_dim, group and chunk sizes
(C/G from 1 to 8, including a non-power of two), context length (ragged tails),
queries per sequence, kept counts and dtype, then runs summaries -> route ->
attend through the C ABI and checks everything against the oracle (exact sets
beyond the score margin, ε-valid choices, outputs within tolerance). Shapes
with many query rows per KV head take the MFMA prefill route, small ones the
one-workgroup-per-row route, the rest the multi-workgroup route. Cases whose
newest queries fit one chunk also run the one-call decode step and compare it
with the separate calls. The last few draw at least 128 queries per sequence in
bf16 with D = 128 and G = 32, so that their attention runs in 128-row tiles
over the union of routed groups (partial last tiles included).
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_summaries_amd as hga
from synth import Workload, generate
from tests.gpu_runner import check_workload, log, run_hip, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 48
N_MANY_ROWS = 4   # the last cases: > 1024 query rows, not the MFMA route
N_TILES = 6       # then: the tile attention


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    if seed >= N_CASES - N_MANY_ROWS:   # multi-workgroup route: f32, or bf16 with r*Nq < 64
        B, Hkv, D = int(rng.integers(2, 4)), 2, int(rng.choice([64, 128]))
        dtype = str(rng.choice(["f32", "bf16"]))
        r, Nq = (8, int(rng.integers(12, 40))) if dtype == "f32" else (1, int(rng.integers(40, 63)))
        Hq = r * Hkv * (1 if dtype == "f32" else 8)
        Hkv = Hkv * (1 if dtype == "f32" else 8)
        G = int(rng.choice([8, 16, 32]))
        C = G * int(rng.choice([2, 4]))
        T = int(rng.integers(max(C, Nq), 2048))
        return Workload(f"random-{seed}", B, Hq, Hkv, D, T, Nq, C, G, int(rng.integers(0, 5)),
                        int(rng.integers(1, 16)), 1e4, dtype, 0)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2]))
    r = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([8, 16, 32]))
    gpc = int(rng.choice([1, 2, 3, 4, 8]))
    C = G * gpc
    T = int(rng.integers(C, 3072))
    Nq = int(rng.choice([1, 2, int(rng.integers(3, 20)), int(rng.integers(20, 90))]))
    Nq = max(1, min(Nq, T))
    k_c = int(rng.integers(0, 7))
    k_g = int(rng.integers(1, 24))
    dtype = str(rng.choice(["bf16", "bf16", "f32"]))
    return Workload(f"random-{seed}", B, r * Hkv, Hkv, D, T, Nq, C, G, k_c, k_g, 1e4, dtype, 0)


def draw_tiles(seed):
    rng = np.random.default_rng(2000 + seed)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2]))
    r = int(rng.choice([1, 2, 4, 8]))
    C = 32 * int(rng.choice([1, 2, 4, 8]))
    Nq = int(rng.integers(128, 401))
    T = int(rng.integers(max(C, Nq), 3072))
    return Workload(f"random-tiles-{seed}", B, r * Hkv, Hkv, 128, T, Nq, C, 32,
                    int(rng.integers(0, 7)), int(rng.integers(1, 24)), 1e4, "bf16", 0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("seed", range(N_CASES + N_TILES))
def test_random_shape(seed):
    w = draw(seed) if seed < N_CASES else draw_tiles(seed - N_CASES)
    log(f"case {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} T={w.T} Nq={w.Nq} "
        f"C={w.chunk} G={w.group} k_c={w.k_chunk} k_g={w.k_group} {w.dtype}")
    inp = generate(w)
    out = run_hip(w, inp)
    check_workload(w, inp, out)
    if w.Nq <= w.chunk:
        Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
        cm, gm = hga.build_summaries(K, w.chunk, w.group)
        O, lse, c_d, g_d = hga.decode_step_ex(Q, K, V, cm, gm, w.T, w.chunk, w.group, w.k_chunk,
                                              w.k_group)
        torch.cuda.synchronize()
        assert torch.equal(g_d, out["gidx"]) and torch.equal(c_d, out["cidx"])
        assert torch.equal(cm, out["cm"]) and torch.equal(gm, out["gm"])
        a, b = O.float(), out["O"].float()
        lim = torch.maximum(a.abs(), b.abs()) * (2.0 ** -7 if w.dtype == "bf16" else 1e-5) + 1e-6
        assert bool(((a - b).abs() <= lim).all())
        assert float((lse - out["lse"]).abs().max()) <= 1e-4
        # the fused refresh-and-route on summaries that are already current
        # rewrites them with the same bits and routes as the separate calls
        cm_f, gm_f = cm.clone(), gm.clone()
        c_f, g_f = hga.route_fresh_ex(Q, K, cm_f, gm_f, w.T, w.chunk, w.group, w.k_chunk,
                                      w.k_group)
        torch.cuda.synchronize()
        assert torch.equal(cm_f, out["cm"]) and torch.equal(gm_f, out["gm"])
        assert torch.equal(g_f, out["gidx"]) and torch.equal(c_f, out["cidx"])

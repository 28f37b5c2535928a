"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes the oracle module and raises AssertionError on a mismatch.
They are called once with the real oracle (test_oracle_pins.py) and again with
deliberately broken copies of it (test_oracle_mutations.py), which each must
trip at least one pin.

Independent sources used here:
  * per-token loops with math.fsum (closed form: the score of a mean key is the
    mean of the per-key scores);
  * brute force over every k-subset (the top-k set is the k-subset with the
    largest score sum, for distinct scores);
  * torch's CPU scaled_dot_product_attention in float64 with an explicit mask
    (dense causal attention, and attention over a gathered token set);
  * the hand-worked fixture tests/golden/hand_worked_tiny.json;
  * invariants the method states: forced first/last chunk, the routed budget.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- summaries
def pin_summary_closed_form(o):
    T, D, C, G = 103, 8, 20, 5            # short last group (3 keys) and chunk (3 keys)
    K = _rand(1, 1, 2, T, D)
    cm, gm = o.build_summaries(K, C, G)
    assert cm.shape == (1, 2, 6, D) and gm.shape == (1, 2, 21, D)
    q = _rand(2, D)
    for h in range(2):
        for g in range(21):
            toks = [j for j in range(T) if j // G == g]
            want = math.fsum(math.fsum(q[d] * K[0, h, j, d] for d in range(D)) for j in toks) / len(toks)
            assert abs(float(gm[0, h, g] @ q) - want) < 1e-12, (h, g)
        for c in range(6):
            toks = [j for j in range(T) if j // C == c]
            want = math.fsum(math.fsum(q[d] * K[0, h, j, d] for d in range(D)) for j in toks) / len(toks)
            assert abs(float(cm[0, h, c] @ q) - want) < 1e-12, (h, c)


# ---------------------------------------------------------------- selection
def _brute_best(ids, scores, k):
    """k-subset of ids with the largest score sum (scores distinct)."""
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(range(len(ids)), k):
        s = math.fsum(scores[t] for t in sub)
        if s > best_sum:
            best, best_sum = sub, s
    return sorted(ids[t] for t in best)


def pin_selection_bruteforce(o):
    T, D, C, G = 64, 4, 8, 2
    per = C // G
    for seed in range(6):
        K = _rand(10 + seed, 1, 1, T, D)
        q = _rand(20 + seed, D)
        cm, gm = o.build_summaries(K, C, G)
        for p, k_c, k_g in [(63, 2, 3), (48, 3, 5), (50, 1, 2), (33, 2, 4)]:
            L = p // C

            def mean_score(toks):
                return math.fsum(float(K[0, 0, j] @ q) for j in toks) / len(toks) / math.sqrt(D)

            cscore = {c: mean_score([j for j in range(T) if j // C == c]) for c in range(L + 1)}
            middle = list(range(1, L))
            if L + 1 <= k_c + 2:
                want_chunks = list(range(L + 1))
            else:
                want_chunks = sorted({0, L, *_brute_best(middle, [cscore[c] for c in middle], k_c)})
            cands = [g for c in want_chunks for g in range(c * per, c * per + per) if g * G <= p]
            gscore = [mean_score([j for j in range(T) if j // G == g]) for g in cands]
            want_groups = sorted(cands) if len(cands) <= k_g else _brute_best(cands, gscore, k_g)
            rq = o.route_query(q, cm[0, 0], gm[0, 0], p, C, G, k_c, k_g)
            assert rq.chunks == want_chunks, (seed, p, rq.chunks, want_chunks)
            assert rq.candidates == cands, (seed, p)
            assert rq.groups == want_groups, (seed, p, rq.groups, want_groups)
            assert np.allclose(rq.chunk_scores, [cscore[c] for c in range(L + 1)], atol=1e-12)


def pin_ties_lower_index(o):
    # Eight identical keys: every chunk and group ties; lower indices must win.
    T, D, C, G = 32, 2, 4, 2
    K = np.ones((1, 1, T, D))
    cm, gm = o.build_summaries(K, C, G)
    rq = o.route_query(np.array([1.0, 0.5]), cm[0, 0], gm[0, 0], 31, C, G, 2, 3)
    assert rq.chunks == [0, 1, 2, 7], rq.chunks
    assert rq.groups == [0, 1, 2], rq.groups
    assert rq.chunk_gap == 0.0 and rq.group_gap == 0.0


def pin_forced_chunks(o):
    # Chunks 0 and L hold keys anti-aligned with q: they score lowest, yet stay.
    T, D, C, G = 128, 4, 16, 4
    K = _rand(5, 1, 1, T, D) * 0.1
    q = np.array([1.0, 0.0, 0.0, 0.0])
    K[0, 0, :C, 0] = -5.0
    K[0, 0, T - C:, 0] = -5.0
    cm, gm = o.build_summaries(K, C, G)
    for k_c in (0, 1, 3):
        rq = o.route_query(q, cm[0, 0], gm[0, 0], T - 1, C, G, k_c, 4)
        assert rq.chunks[0] == 0 and rq.chunks[-1] == T // C - 1, rq.chunks
        assert len(rq.chunks) == k_c + 2
        if k_c == 0:
            assert rq.chunks == [0, T // C - 1]
    # The query's own chunk, not the cache's last, is forced when p < T-1.
    rq = o.route_query(q, cm[0, 0], gm[0, 0], 70, C, G, 1, 4)
    assert rq.chunks[0] == 0 and rq.chunks[-1] == 70 // C


# ---------------------------------------------------------------- attention
def _sdpa(q, k, v, mask, scale):
    """torch CPU float64 attention; q [1,H,Nq,D], k/v [1,H,T,D], mask [Nq,T] bool."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()


def pin_all_selected_is_dense(o):
    B, Hq, Hkv, Nq, T, D, C, G = 1, 4, 2, 5, 96, 8, 16, 4
    Q = _rand(30, B, Hq, Nq, D)
    K = _rand(31, B, Hkv, T, D)
    V = _rand(32, B, Hkv, T, D)
    cm, gm = o.build_summaries(K, C, G)
    _, gidx, _ = o.route(Q, cm, gm, T, C, G, k_chunk=T // C, k_group=T // G)
    O, lse = o.attend(Q, K, V, gidx, G)
    Od, lsed = o.dense_causal(Q, K, V)
    # bottom-right causal mask: query i sits at position T - Nq + i
    mask = np.arange(T)[None, :] <= (T - Nq + np.arange(Nq))[:, None]
    Kr = np.repeat(K, Hq // Hkv, axis=1)     # consecutive query heads share a KV head
    Vr = np.repeat(V, Hq // Hkv, axis=1)
    ref = _sdpa(Q, Kr, Vr, mask, 1.0 / math.sqrt(D))
    assert np.abs(O - ref).max() < 1e-12, np.abs(O - ref).max()
    assert np.abs(Od - ref).max() < 1e-12
    logits = np.einsum("bhnd,bhtd->bhnt", Q, Kr) / math.sqrt(D)
    logits = np.where(mask[None, None], logits, -np.inf)
    lref = torch.logsumexp(torch.from_numpy(logits), dim=-1).numpy()
    assert np.abs(lse - lref).max() < 1e-12 and np.abs(lsed - lref).max() < 1e-12
    # an explicit scale is honoured
    O2, _ = o.dense_causal(Q, K, V, scale=0.3)
    assert np.abs(O2 - _sdpa(Q, Kr, Vr, mask, 0.3)).max() < 1e-12


def pin_attend_on_gathered_set(o):
    B, Hq, Hkv, Nq, T, D, G = 1, 2, 1, 3, 80, 8, 8
    Q = _rand(40, B, Hq, Nq, D)
    K = _rand(41, B, Hkv, T, D)
    V = _rand(42, B, Hkv, T, D)
    gidx = np.full((B, Hq, Nq, 4), -1, dtype=np.int32)
    sets = {(0, 0): [1, 4, 9], (0, 1): [0, 9], (0, 2): [2, 3, 5, 9],
            (1, 0): [7], (1, 1): [3, 8], (1, 2): [0, 1, 2, 6]}
    for (h, i), gs in sets.items():
        gidx[0, h, i, :len(gs)] = gs
    O, lse = o.attend(Q, K, V, gidx, G)
    for (h, i), gs in sets.items():
        p = T - Nq + i
        toks = torch.cat([torch.arange(g * G, (g + 1) * G) for g in gs])
        toks = toks[toks <= p].numpy()
        ref = _sdpa(Q[:, h:h + 1, i:i + 1], K[:, :, toks], V[:, :, toks],
                    np.ones((1, len(toks)), dtype=bool), 1.0 / math.sqrt(D))
        assert np.abs(O[0, h, i] - ref[0, 0, 0]).max() < 1e-12, (h, i)
        lg = torch.from_numpy(K[0, 0, toks] @ Q[0, h, i] / math.sqrt(D))
        assert abs(lse[0, h, i] - float(torch.logsumexp(lg, 0))) < 1e-12


def pin_causality(o):
    # With the routed groups fixed, keys/values after p cannot change query p.
    B, Hq, Hkv, Nq, T, D, G = 1, 1, 1, 4, 40, 4, 8
    Q = _rand(50, B, Hq, Nq, D)
    K = _rand(51, B, Hkv, T, D)
    V = _rand(52, B, Hkv, T, D)
    gidx = np.array([[[[0, 4], [2, 4], [4, -1], [1, 4]]]], dtype=np.int32)
    O1, l1 = o.attend(Q, K, V, gidx, G)
    K2, V2 = K.copy(), V.copy()
    K2[:, :, T - Nq + 1:] += 7.0
    V2[:, :, T - Nq + 1:] -= 3.0
    O2, l2 = o.attend(Q, K2, V2, gidx, G)
    assert np.array_equal(O1[..., 0, :], O2[..., 0, :]) and l1[..., 0] == l2[..., 0]
    assert not np.allclose(O1[..., 3, :], O2[..., 3, :])


# ---------------------------------------------------------------- worked example
def pin_hand_worked_example(o):
    with open(os.path.join(GOLDEN, "hand_worked_tiny.json")) as f:
        ex = json.load(f)
    T, D, C, G, p = ex["T"], ex["D"], ex["chunk"], ex["group"], ex["p"]
    K = np.zeros((1, 1, T, D))
    K[0, 0, :, 0] = ex["key_x"]
    K[0, 0, :, 1] = ex["key_y"]
    V = np.zeros((1, 1, T, D))
    for j in range(T):
        V[0, 0, j] = ex["value"].get(str(j), ex["value"]["default"])
    env = {"e": math.e, "log": math.log, "sqrt": math.sqrt}
    q = np.array([eval(s, env) for s in ex["q"]])
    cm, gm = o.build_summaries(K, C, G)
    for case in ex["cases"]:
        rq = o.route_query(q, cm[0, 0], gm[0, 0], p, C, G, case["k_chunk"], case["k_group"])
        assert np.allclose(rq.chunk_scores, ex["expected_chunk_scores"], atol=1e-12, rtol=0)
        assert rq.chunks == case["chunks"], (rq.chunks, case)
        assert rq.candidates == case["candidates"]
        assert np.allclose(rq.cand_scores, case["candidate_scores"], atol=1e-12, rtol=0)
        assert rq.groups == case["groups"], (rq.groups, case)
        assert math.isclose(rq.chunk_gap, float(case["chunk_gap"]), abs_tol=1e-12)
        assert math.isclose(rq.group_gap, float(case["group_gap"]), abs_tol=1e-12)
        assert o.routed_tokens(rq.groups, G, p, T) == case["tokens"]
        gidx = np.array(rq.groups, dtype=np.int32).reshape(1, 1, 1, -1)
        O, lse = o.attend(q.reshape(1, 1, 1, D), K, V, gidx, G)
        want = [eval(case["out_x"], env), eval(case["out_y"], env)]
        assert np.allclose(O[0, 0, 0], want, atol=1e-12, rtol=0), (O[0, 0, 0], want)
        assert math.isclose(lse[0, 0, 0], eval(case["lse"], env), abs_tol=1e-12)


# ---------------------------------------------------------------- generator invariants
def pin_budget_and_planting(o):
    """On a planted long-context workload: every query keeps exactly
    k_group*group tokens (the configured sparsity), its planted chunks are all
    retrieved, and its groups all come from its planted chunks."""
    from synth import DECODE_64K, generate, plant_count
    w = DECODE_64K.with_(T=16384, k_chunk=8, k_group=16, Hq=16, Hkv=2)
    inp = generate(w, seed=0)
    cm, gm = o.build_summaries(inp.K, w.chunk, w.group)
    cidx, gidx, rec = o.route(inp.Q, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group)
    P = plant_count(w)
    assert P == 7
    per = w.chunk // w.group
    for (b, h, i), rq in rec.items():
        toks = o.routed_tokens(rq.groups, w.group, w.T - 1, w.T)
        assert len(toks) == w.k_group * w.group
        planted = inp.planted[(b, h)]
        assert set(planted) <= set(rq.chunks), (h, planted, rq.chunks)
        assert all(g // per in planted for g in rq.groups)
        assert len(rq.chunks) == w.k_chunk + 2


PINS = [pin_summary_closed_form, pin_selection_bruteforce, pin_ties_lower_index,
        pin_forced_chunks, pin_all_selected_is_dense, pin_attend_on_gathered_set,
        pin_causality, pin_hand_worked_example, pin_budget_and_planting]

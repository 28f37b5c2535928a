"""The seeded input generator: determinism, rounding, RoPE and planting facts."""
import numpy as np
import torch

from synth import DECODE_64K, TINY, generate, gen_kv_slice, gen_q, plant_count, rope, round_to_dtype


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [0.0, -0.0, 1.00390625, 1.01171875]      # exact ties between bf16 neighbours
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(round_to_dtype(x, "bf16"), want)


def test_rope_is_a_rotation():
    x = np.random.default_rng(1).standard_normal((50, 64))
    pos = np.arange(50) * 37
    y = rope(x, pos, 1e4)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1))
    assert np.allclose(rope(x[:1], np.array([0]), 1e4), x[:1])
    # relative-position property: <R_a q, R_b k> depends only on b - a
    q, k = x[0], x[1]
    d1 = rope(q[None], np.array([5]), 1e4) @ rope(k[None], np.array([9]), 1e4).T
    d2 = rope(q[None], np.array([105]), 1e4) @ rope(k[None], np.array([109]), 1e4).T
    assert np.allclose(d1, d2)


def test_deterministic_and_slice_independent():
    w = DECODE_64K.with_(T=4096, k_chunk=2, k_group=4)
    a = generate(w, seed=3)
    Q = gen_q(w, seed=3)
    k, v, pl = gen_kv_slice(w, 3, 0, 2, Q)
    assert np.array_equal(a.Q, Q)
    assert np.array_equal(a.K[0, 2], k) and np.array_equal(a.V[0, 2], v)
    assert all(a.planted[(0, h)] == pl[h] for h in pl)
    b = generate(w, seed=4)
    assert not np.array_equal(a.K, b.K)


def test_planted_keys_are_query_aligned():
    w = DECODE_64K.with_(T=16384, k_chunk=8, k_group=16)
    inp = generate(w, seed=0)
    assert plant_count(w) == 7
    for (b, h), chunks in inp.planted.items():
        assert len(chunks) == 7 and 0 not in chunks and w.n_chunks - 1 not in chunks
        qh = inp.Q[b, h, -1].astype(np.float64)
        qh /= np.linalg.norm(qh)
        kk = inp.K[b, h // w.r, chunks[0] * w.chunk:(chunks[0] + 1) * w.chunk].astype(np.float64)
        cos = kk @ qh / np.linalg.norm(kk, axis=1)
        assert np.allclose(cos, 0.6, atol=5e-3)        # exact before bf16 rounding
    # disjoint across the query heads of one KV head
    for kv in range(w.Hkv):
        seen = [c for h in range(kv * w.r, (kv + 1) * w.r) for c in inp.planted[(0, h)]]
        assert len(seen) == len(set(seen))


def test_tiny_is_fp32_and_unplanted():
    inp = generate(TINY)
    assert inp.planted == {} and inp.Q.dtype == np.float32
    assert not np.array_equal(round_to_dtype(inp.K, "bf16"), inp.K)

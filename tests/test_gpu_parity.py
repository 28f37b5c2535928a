"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Workloads: the tiny fp32 case and its all-selected twin (which must equal dense
causal attention), the 64K-context Qwen3-30B-A3B-shaped decode layer, the
batch-16 context sweep, and edge shapes (ragged T, short and single chunks,
k_chunk 0, padding, every position a query, MHA, r = 16, D = 64, G > 32).
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_summaries_amd as hga
import oracle
from synth import DECODE_64K, HOST_TIER, PREFILL, SWEEP, TINY, TINY_ALL, Workload, generate
from tests import parity
from tests.gpu_runner import check_sampled, check_workload, log, np_of, run_hip, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def test_tiny_f32():
    log("case tiny-f32")
    inp = generate(TINY)
    out = run_hip(TINY, inp)
    check_workload(TINY, inp, out)


def test_tiny_all_selected_equals_dense():
    log("case tiny-f32 all-selected")
    inp = generate(TINY_ALL)
    out = run_hip(TINY_ALL, inp)
    check_workload(TINY_ALL, inp, out)
    Od, lsed = oracle.dense_causal(inp.Q, inp.K, inp.V)
    parity.check_outputs(np_of(out["O"]), np_of(out["lse"]), Od, lsed, "f32")
    gidx = out["gidx"].cpu().numpy()
    for i in range(TINY.Nq):   # every group up to the query's own is routed
        p = TINY.T - TINY.Nq + i
        assert [g for g in gidx[0, 0, i] if g >= 0] == list(range(p // TINY.group + 1))


EDGE = [
    # ragged T (partial last chunk and group), planted, B=2
    Workload("edge-ragged", 2, 8, 2, 128, 5000, 1, 256, 32, 4, 12, 1e6, "bf16", 2),
    # D=64 bf16, MHA, 3 queries with straddling groups
    Workload("edge-d64-mha", 1, 4, 4, 64, 3000, 3, 128, 16, 3, 10, 1e4, "bf16", 0),
    # fp32, r=16 (two 16-row blocks per KV head at Nq=2)
    Workload("edge-f32-r16", 1, 16, 1, 128, 2048, 2, 64, 8, 5, 20, 1e4, "f32", 0),
    # fewer keys than one chunk: only chunk 0 exists
    Workload("edge-single-chunk", 1, 2, 1, 128, 200, 1, 256, 32, 4, 3, 1e4, "bf16", 0),
    # no chunk picked by score: only the forced ones
    Workload("edge-kc0", 1, 8, 2, 128, 4096, 1, 256, 32, 0, 6, 1e6, "bf16", 0),
    # fewer candidates than k_group: -1 padding
    Workload("edge-pad", 1, 4, 1, 128, 1024, 1, 256, 64, 1, 20, 1e4, "bf16", 0),
    # every position is a query (p = 0 included)
    Workload("edge-all-positions", 1, 2, 1, 64, 100, 100, 32, 8, 2, 3, 1e4, "f32", 0),
    # group == chunk, and groups of 64 tokens (two gather tiles)
    Workload("edge-gpc1-g64", 1, 8, 1, 128, 4096, 1, 64, 64, 6, 6, 1e6, "bf16", 0),
    # groups of 48 tokens (a partial second tile)
    Workload("edge-g48", 1, 4, 2, 128, 3000, 2, 96, 48, 5, 7, 1e4, "bf16", 0),
]


# Many query rows per KV head (r * Nq >= 64, bf16): MFMA scoring + select kernel.
PREFILL_SMALL = [
    Workload("prefill-small", 1, 8, 2, 128, 4096, 100, 128, 32, 4, 8, 1e6, "bf16", 2),
    Workload("prefill-d64-ragged", 2, 4, 1, 64, 2000, 64, 64, 16, 6, 10, 1e4, "bf16", 0),
    Workload("prefill-gpc1-mha", 1, 2, 2, 128, 1500, 70, 32, 32, 5, 5, 1e4, "bf16", 0),
    # C/G not a power of two: the three-kernel form (scores through the workspace)
    Workload("prefill-gpc3", 1, 8, 2, 128, 3000, 100, 96, 32, 4, 8, 1e4, "bf16", 0),
]


# Query rows in tiles of 128 per head (bf16, D 128, G 32): the prefill
# attention runs on MFMA over each tile's union of routed groups. Full tiles
# and a partial last tile; one tile exactly, with B = 2 and one query head per
# KV head.
PREFILL_TILES = [
    Workload("prefill-tiles-nq300", 1, 8, 2, 128, 4096, 300, 128, 32, 4, 8, 1e6, "bf16", 2),
    Workload("prefill-tiles-b2-mha", 2, 2, 2, 128, 2048, 128, 64, 32, 5, 6, 1e4, "bf16", 0),
]


# More than 1024 query rows without the MFMA path: the multi-workgroup route
# (dense scoring of a KV head's summaries, last-arriving workgroup selects).
FUSED_ROUTE = [
    Workload("fused-f32-rows1600", 1, 8, 8, 128, 2048, 200, 64, 16, 5, 9, 1e4, "f32", 0),
    Workload("fused-bf16-b40-decode", 40, 32, 4, 128, 4096, 1, 256, 32, 2, 4, 1e6, "bf16", 1),
]


@pytest.mark.parametrize("w", FUSED_ROUTE, ids=lambda w: w.name)
def test_fused_route_many_rows(w):
    log(f"case {w.name}")
    inp = generate(w)
    out = run_hip(w, inp)
    check_workload(w, inp, out)


@pytest.mark.parametrize("w", PREFILL_SMALL, ids=lambda w: w.name)
def test_prefill_small(w):
    log(f"case {w.name}")
    inp = generate(w)
    out = run_hip(w, inp)
    check_workload(w, inp, out)


@pytest.mark.parametrize("w", PREFILL_TILES, ids=lambda w: w.name)
def test_prefill_tiles(w):
    log(f"case {w.name}")
    inp = generate(w)
    out = run_hip(w, inp)
    check_workload(w, inp, out)


def test_prefill_4096_on_61440_sampled():
    w = PREFILL
    log(f"case {w.name}")
    inp = generate(w)
    out = run_hip(w, inp)
    check_sampled(w, inp, out, n_rows=256)
    # the last new token of every head retrieves its planted chunks
    gidx = out["gidx"].cpu().numpy()
    per = w.chunk // w.group
    for h in range(w.Hq):
        assert sorted(set(g // per for g in gidx[0, h, -1])) == inp.planted[(0, h)]
    # the prefill step the benchmark times (refresh of the new keys' chunks,
    # routing, attention) against the sampled-and-checked separate calls
    cm, gm = hga.build_summaries(out["K"], w.chunk, w.group)
    O, lse, c_d, g_d = hga.decode_step_ex(out["Q"], out["K"], out["V"], cm, gm, w.T, w.chunk,
                                          w.group, w.k_chunk, w.k_group)
    torch.cuda.synchronize()
    assert torch.equal(cm, out["cm"]) and torch.equal(gm, out["gm"])
    assert torch.equal(g_d, out["gidx"]) and torch.equal(c_d, out["cidx"])
    _same_attention(O, lse, out["O"], out["lse"], w.dtype)


def test_host_tier_b4_t262144_sampled():
    """Full K/V in pinned host memory, summaries in HBM: the routed groups are
    read over the host link. Every one of the workload's 128 query rows
    against the oracle (the per-row oracle path of the sampled check)."""
    w = HOST_TIER
    log(f"case {w.name}")
    inp = generate(w)
    out = run_hip(w, inp)
    assert not out["K"].is_cuda and out["cm"].is_cuda
    rows = w.B * w.Hq * w.Nq
    st, _ = check_sampled(w, inp, out, n_rows=rows)
    assert st.queries == rows == 128


@pytest.mark.parametrize("w", EDGE, ids=lambda w: w.name)
def test_edge_shapes(w):
    log(f"case {w.name}")
    inp = generate(w)
    out = run_hip(w, inp)
    check_workload(w, inp, out)


def test_qwen3_decode_64k():
    w = DECODE_64K
    log(f"case {w.name}")
    inp = generate(w)
    out = run_hip(w, inp)
    st, _ = check_workload(w, inp, out)
    # planted chunks are retrieved and fill the group budget: 64 groups = 2048 tokens (3.125%)
    gidx = out["gidx"].cpu().numpy()
    per = w.chunk // w.group
    for h in range(w.Hq):
        planted = inp.planted[(0, h)]
        assert sorted(set(g // per for g in gidx[0, h, 0])) == planted
        assert (gidx[0, h, 0] >= 0).sum() == w.k_group


@pytest.mark.parametrize("T", sorted(SWEEP))
def test_sweep_b16(T):
    """Every sequence of the batch-16 sweep point: the decode step the
    benchmark times (refreshing route, then attention) against the oracle
    element by element, and the three separate calls against the decode step
    (summaries and routes bit for bit, attention to fp32 rounding)."""
    w = SWEEP[T]
    log(f"case {w.name}")
    inp = generate(w)
    out = run_hip(w, inp)
    Q, K, V = out["Q"], out["K"], out["V"]
    cm, gm = hga.build_summaries(K, w.chunk, w.group)
    O, lse, c_d, g_d = hga.decode_step_ex(Q, K, V, cm, gm, w.T, w.chunk, w.group, w.k_chunk,
                                          w.k_group)
    torch.cuda.synchronize()
    check_workload(w, inp, dict(cm=cm, gm=gm, cidx=c_d, gidx=g_d, O=O, lse=lse))
    assert torch.equal(cm, out["cm"]) and torch.equal(gm, out["gm"])
    assert torch.equal(g_d, out["gidx"]) and torch.equal(c_d, out["cidx"])
    _same_attention(O, lse, out["O"], out["lse"], w.dtype)


def test_update_summaries_bit_identical_to_build():
    log("case update-summaries")
    w = DECODE_64K.with_(T=5000, B=2)
    inp = generate(w)
    K = to_dev(inp.K, w.dtype)
    cm, gm = hga.build_summaries(K, w.chunk, w.group)
    # change keys in one place, refresh only there, compare with a full rebuild
    K[:, :, 4100:4103] += 1.5
    hga.update_summaries(K, w.chunk, w.group, 4100, 4103, cm, gm)
    cm2, gm2 = hga.build_summaries(K, w.chunk, w.group)
    torch.cuda.synchronize()
    assert torch.equal(cm, cm2) and torch.equal(gm, gm2)
    # appending the last key of the cache
    K[:, :, -1] -= 2.0
    hga.update_summaries(K, w.chunk, w.group, w.T - 1, w.T, cm, gm)
    cm2, gm2 = hga.build_summaries(K, w.chunk, w.group)
    torch.cuda.synchronize()
    assert torch.equal(cm, cm2) and torch.equal(gm, gm2)


def test_deterministic():
    log("case determinism")
    w = DECODE_64K.with_(T=16384, k_chunk=8, k_group=16, B=2)
    inp = generate(w)
    a = run_hip(w, inp)
    b = run_hip(w, inp)
    for k in ("cm", "gm", "cidx", "gidx", "O", "lse"):
        assert torch.equal(a[k], b[k]), k


def test_explicit_scale():
    log("case explicit-scale")
    w = DECODE_64K.with_(T=4096, k_chunk=4, k_group=8)
    inp = generate(w)
    out = run_hip(w, inp, scale=0.05)
    check_workload(w, inp, out, scale=0.05)


@pytest.mark.parametrize("path", ["decode-step", "prefill-tiles", "many-row-route"])
def test_explicit_scale_every_path(path):
    """A caller's scale reaches every path that applies it itself: the
    one-launch decode step, the prefill MFMA route with the tile attention, and
    the many-row route; each against the oracle at that scale."""
    s = 0.05
    log(f"case explicit-scale {path}")
    if path == "decode-step":
        w = DECODE_64K.with_(T=4096, k_chunk=4, k_group=8)
        shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
        assert hga.decode_step_one_launch(shape, w.dtype, w.chunk, w.group, w.k_chunk, w.k_group)
        inp = generate(w)
        Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
        cm, gm = hga.build_summaries(K, w.chunk, w.group)
        O, lse, c_d, g_d = hga.decode_step_ex(Q, K, V, cm, gm, w.T, w.chunk, w.group, w.k_chunk,
                                              w.k_group, scale=s)
        torch.cuda.synchronize()
        out = dict(cm=cm, gm=gm, cidx=c_d, gidx=g_d, O=O, lse=lse)
    else:
        w = PREFILL_TILES[0] if path == "prefill-tiles" else FUSED_ROUTE[0]
        inp = generate(w)
        out = run_hip(w, inp, scale=s)
    check_workload(w, inp, out, scale=s)


def test_default_workspaces_are_per_stream():
    """Attention calls on two streams at once, each with the binding's default
    workspace (rows split over two workgroups joined by arrival counters in the
    workspace): each stream gets a workspace of its own, so the results equal
    those of the same calls made one after another."""
    log("case per-stream workspaces")
    w = DECODE_64K.with_(B=2, T=8192, k_chunk=4, k_group=8)
    shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
    # split rows: their partials take workspace beyond the zero region
    assert hga.attend_workspace_bytes(shape, w.group, w.k_group) > hga.WORKSPACE_ZERO_BYTES
    inp = generate(w)
    out = run_hip(w, inp)
    Q, K, V, g = out["Q"], out["K"], out["V"], out["gidx"]
    Q2 = -Q
    O_a, l_a = hga.attend(Q, K, V, g, w.group)
    O_b, l_b = hga.attend(Q2, K, V, g, w.group)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    res = []
    for _ in range(10):
        with torch.cuda.stream(s1):
            r1 = hga.attend(Q, K, V, g, w.group)
        with torch.cuda.stream(s2):
            r2 = hga.attend(Q2, K, V, g, w.group)
        res.append((r1, r2))
    torch.cuda.synchronize()
    for (O1, l1), (O2, l2) in res:
        assert torch.equal(O1, O_a) and torch.equal(l1, l_a)
        assert torch.equal(O2, O_b) and torch.equal(l2, l_b)


@pytest.mark.parametrize("case", ["b1-one-launch", "b16-two-launches", "noalloc", "prefill"])
def test_decode_step_graph_replays_match_eager(case):
    """The decode step captured in a HIP graph, as the benchmark times it, and
    replayed several times with other calls and synchronizations in between:
    every replay's outputs equal the eager call's. The workspace's zero region
    is therefore back at zero after each replay; the library clears it with a
    fill kernel, never a memset node. The allocation-free entry point (the one
    for callers under capture) is captured the same way."""
    log(f"case graph replays {case}")
    w = {"b16-two-launches": SWEEP[4096], "prefill": PREFILL_TILES[0]}.get(
        case, DECODE_64K.with_(T=8192, k_chunk=4, k_group=8))
    inp = generate(w)
    Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
    cm, gm = hga.build_summaries(K, w.chunk, w.group)
    shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
    one = hga.decode_step_one_launch(shape, w.dtype, w.chunk, w.group, w.k_chunk, w.k_group)
    assert one == (case not in ("b16-two-launches", "prefill"))
    ws = torch.zeros(hga.decode_step_workspace_bytes(shape, w.chunk, w.group, w.k_chunk,
                                                     w.k_group), dtype=torch.uint8, device="cuda")
    O = torch.empty_like(Q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    gidx = torch.empty((w.B, w.Hq, w.Nq, w.k_group), dtype=torch.int32, device="cuda")
    cidx = torch.empty((w.B, w.Hq, w.Nq, w.k_chunk + 2), dtype=torch.int32, device="cuda")

    def step():
        if case == "noalloc":
            hga.decode_step_noalloc(Q, K, V, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                                    chunk_idx=cidx, group_idx=gidx, out=O, lse=lse)
        else:
            hga.decode_step_ex(Q, K, V, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                               chunk_idx=cidx, group_idx=gidx, out=O, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (O, lse, gidx, cidx, cm, gm)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                      # once on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(4):
        for t in (O, lse):
            t.zero_()
        gidx.fill_(-5)
        cidx.fill_(-5)
        hga.attend(Q, K, V, want[2], w.group)      # other work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip((O, lse, gidx, cidx, cm, gm), want):
            assert torch.equal(got, ref)
    if case != "noalloc":
        hga.workspace_check(ws)     # no bounded wait gave up


def test_kv_in_pinned_host_memory():
    log("case pinned-host-kv")
    w = DECODE_64K.with_(T=8192, k_chunk=4, k_group=8, B=2)
    inp = generate(w)
    out = run_hip(w, inp)
    Kh = torch.from_numpy(inp.K).to(torch.bfloat16).pin_memory()
    Vh = torch.from_numpy(inp.V).to(torch.bfloat16).pin_memory()
    O, lse = hga.attend(out["Q"], Kh, Vh, out["gidx"], w.group)
    torch.cuda.synchronize()
    assert torch.equal(O, out["O"]) and torch.equal(lse, out["lse"])


def test_back_to_back_calls_share_workspace():
    """Two different inputs of one shape through the same workspaces, with no
    synchronisation between them: the second call must not see the first
    call's cross-workgroup partials or scores."""
    log("case back-to-back")
    w = DECODE_64K.with_(T=16384, k_chunk=8, k_group=16)
    a = generate(w, seed=11)
    b = generate(w, seed=12)
    Qa, Ka, Va = (to_dev(x, w.dtype) for x in (a.Q, a.K, a.V))
    Qb, Kb, Vb = (to_dev(x, w.dtype) for x in (b.Q, b.K, b.V))
    cma, gma = hga.build_summaries(Ka, w.chunk, w.group)
    cmb, gmb = hga.build_summaries(Kb, w.chunk, w.group)
    outs = []
    for Q, K, V, cm, gm in ((Qa, Ka, Va, cma, gma), (Qb, Kb, Vb, cmb, gmb), (Qa, Ka, Va, cma, gma)):
        cidx, gidx = hga.route(Q, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group)
        O, lse = hga.attend(Q, K, V, gidx, w.group)
        outs.append(dict(Q=Q, cm=cm, gm=gm, cidx=cidx, gidx=gidx, O=O, lse=lse))
    torch.cuda.synchronize()
    check_workload(w, a, outs[0])
    check_workload(w, b, outs[1])
    check_workload(w, a, outs[2])
    assert torch.equal(outs[0]["O"], outs[2]["O"])


def test_quality_proxy_matches_oracle():
    """Share of the dense softmax mass on the routed tokens, from the library's
    attention over all groups vs over the routed groups, against the oracle's
    dense and routed log-sum-exp."""
    log("case quality-proxy")
    w = DECODE_64K.with_(T=16384, k_chunk=8, k_group=16, B=2)
    inp = generate(w)
    out = run_hip(w, inp)
    all_g = torch.arange(w.n_groups, dtype=torch.int32, device="cuda")
    all_g = all_g.expand(w.B, w.Hq, w.Nq, w.n_groups).contiguous()
    Od, lsed = hga.attend(out["Q"], out["K"], out["V"], all_g, w.group)
    torch.cuda.synchronize()
    mass_gpu = torch.exp(out["lse"] - lsed).cpu().numpy()
    Od_ref, lsed_ref = oracle.dense_causal(inp.Q, inp.K, inp.V)
    parity.check_outputs(np_of(Od), lsed.cpu().numpy(), Od_ref, lsed_ref, w.dtype)
    _, lser_ref = oracle.attend(inp.Q, inp.K, inp.V, out["gidx"].cpu().numpy(), w.group)
    mass_ref = np.exp(lser_ref - lsed_ref)
    assert np.abs(mass_gpu - mass_ref).max() < 2e-3 * max(1.0, mass_ref.max())
    assert (mass_ref > 0).all() and (mass_ref <= 1 + 1e-9).all()   # a share of the dense mass


def _ragged_case(Nq=1):
    w = DECODE_64K.with_(name="ragged-b4-t8192", B=4, Hq=8, Hkv=2, T=8192, Nq=Nq, k_chunk=4,
                         k_group=12, plants=2)
    inp = generate(w)
    seq_lens = [8192, 5000, 1234, 3001]
    return w, inp, seq_lens


def _run_ragged(w, inp, seq_lens, layout, K, V):
    Q = to_dev(inp.Q, w.dtype)
    cm, gm = hga.build_summaries_ex(K, w.chunk, w.group, layout=layout, seq_len=w.T)
    cidx, gidx = hga.route_ex(Q, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group, layout=layout)
    O, lse = hga.attend_ex(Q, K, V, gidx, w.group, layout=layout, seq_len=w.T)
    torch.cuda.synchronize()
    return dict(Q=Q, cm=cm, gm=gm, cidx=cidx, gidx=gidx, O=O, lse=lse)


def _pages(w, inp, seq_lens, page_tokens, seed=5):
    """The same caches cut into pages of page_tokens, scattered over a pool in a
    random order; unused block-table entries are -1."""
    rng = np.random.default_rng(seed)
    need = [-(-int(t) // page_tokens) for t in seq_lens]
    n_pages = sum(need) + 3
    order = rng.permutation(n_pages)
    max_pages = -(-w.T // page_tokens)
    table = np.full((w.B, max_pages), -1, dtype=np.int32)
    kp = np.zeros((n_pages, w.Hkv, page_tokens, w.D), dtype=np.float32)
    vp = np.zeros_like(kp)
    k = 0
    for b in range(w.B):
        for j in range(need[b]):
            pid = int(order[k]); k += 1
            table[b, j] = pid
            seg = slice(j * page_tokens, (j + 1) * page_tokens)   # the last may be partial
            n = inp.K[b, :, seg].shape[1]
            kp[pid, :, :n] = inp.K[b, :, seg]
            vp[pid, :, :n] = inp.V[b, :, seg]
    return (to_dev(kp, w.dtype), to_dev(vp, w.dtype),
            torch.from_numpy(table).cuda(), n_pages)


@pytest.mark.parametrize("Nq", [1, 2])
def test_ragged_dense_cache(Nq):
    log(f"case ragged-dense Nq={Nq}")
    w, inp, seq_lens = _ragged_case(Nq)
    lens = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    layout = hga.Layout(seq_lens=lens)
    out = _run_ragged(w, inp, seq_lens, layout, to_dev(inp.K, w.dtype), to_dev(inp.V, w.dtype))
    from tests.gpu_runner import check_ragged
    check_ragged(w, inp, seq_lens, out)


def _ids_with_strays(w, rng):
    """Per row: up to 9 distinct groups at or before the row's position (its
    own group, partly after it, always among them), then ids no group has:
    n_g, n_g + 7 and -5."""
    n_g = -(-w.T // w.group)
    gidx = np.full((w.B, w.Hq, w.Nq, w.k_group), -1, dtype=np.int32)
    for b in range(w.B):
        for h in range(w.Hq):
            for i in range(w.Nq):
                own = (w.T - w.Nq + i) // w.group
                pick = rng.choice(own, size=min(8, own), replace=False) if own > 0 else []
                ids = [own, *[int(x) for x in pick], n_g, n_g + 7, -5]
                gidx[b, h, i, :len(ids)] = ids[:w.k_group]
    return gidx


@pytest.mark.parametrize("nq", [1, 160])
def test_attend_ignores_ids_and_pages_out_of_range(nq):
    """Group ids outside [0, n_g), and routed groups whose page id lies outside
    the pool, contribute nothing: the outputs equal the oracle's attention over
    the other groups, on a dense and on a paged cache, and staged attention
    equals the direct one. Nq = 1 runs the per-row gather, Nq = 160 the tile
    attention (bf16, D 128, G 32); both read a group's rows through a range
    that ends where its valid rows end."""
    log(f"case out-of-range ids and pages Nq={nq}")
    w = Workload(f"stray-ids-nq{nq}", 1, 4, 2, 128, 2000, nq, 128, 32, 4, 12, 1e4, "bf16", 0)
    inp = generate(w)
    gidx_np = _ids_with_strays(w, np.random.default_rng(11))
    # a few rows of head 1 list stray ids only: no token, so O = 0, lse = -inf
    empty = [i for i in (0, 77, nq - 1) if i < nq]
    ids_empty = gidx_np.copy()
    ids_empty[0, 1, empty] = -1
    ids_empty[0, 1, empty, :3] = [-(2 ** 31), 10 ** 6, -3]
    Q = to_dev(inp.Q, w.dtype)

    def check(O, lse, ids_ref):
        O, lse = np_of(O), lse.cpu().numpy()
        assert (O[0, 1, empty] == 0).all() and np.isneginf(lse[0, 1, empty]).all()
        O_ref, lse_ref = oracle.attend(inp.Q, inp.K, inp.V, ids_ref, w.group)
        O_ref[0, 1, empty] = 0
        lse[0, 1, empty] = lse_ref[0, 1, empty] = 0
        parity.check_outputs(O, lse, O_ref, lse_ref, w.dtype)

    gidx = torch.from_numpy(ids_empty).cuda()
    K, V = to_dev(inp.K, w.dtype), to_dev(inp.V, w.dtype)
    O, lse = hga.attend(Q, K, V, gidx, w.group)
    torch.cuda.synchronize()
    check(O, lse, gidx_np)   # the oracle sees the empty rows' original ids (it needs a token)
    # staged attention (routed groups copied into a pool first) ignores them alike
    O3, lse3 = hga.attend_staged(Q, K, V, gidx, w.group)
    torch.cuda.synchronize()
    assert torch.equal(O3, O) and torch.equal(lse3, lse)

    # paged: pages 3 and 10 point past the pool, page 20 before it
    page_tokens = 64
    kp, vp, table, n_pages = _pages(w, inp, [w.T], page_tokens)
    bad = {3: n_pages + 3, 10: n_pages, 20: -2}
    for j, pid in bad.items():
        table[0, j] = pid
    layout = hga.Layout(block_table=table, page_tokens=page_tokens, n_pages=n_pages)
    O2, lse2 = hga.attend_ex(Q, kp, vp, gidx, w.group, layout=layout, seq_len=w.T)
    torch.cuda.synchronize()
    per = page_tokens // w.group
    gone = np.isin(gidx_np // per, list(bad)) & (gidx_np >= 0)
    check(O2, lse2, np.where(gone, -1, gidx_np))


@pytest.mark.parametrize("nq", [1, 160])
def test_seq_lens_are_clamped(nq):
    """Per-sequence lengths past T, or negative, act as T and 0 in every call:
    summaries, routing, attention and the decode step equal those of the
    clamped lengths bit for bit (Nq = 160 takes the MFMA route and the tile
    attention)."""
    log(f"case clamped seq_lens Nq={nq}")
    w = Workload(f"clamp-nq{nq}", 3, 8, 2, 128, 2048, nq, 128, 32, 4, 8, 1e4, "bf16", 0)
    inp = generate(w)
    Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
    n_c, n_g = hga.summary_counts(w.T, w.chunk, w.group)

    def run(lens):
        layout = hga.Layout(seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
        cm = torch.zeros((w.B, w.Hkv, n_c, w.D), dtype=torch.float32, device="cuda")
        gm = torch.zeros((w.B, w.Hkv, n_g, w.D), dtype=torch.float32, device="cuda")
        hga.build_summaries_ex(K, w.chunk, w.group, layout=layout, seq_len=w.T,
                               chunk_mean=cm, group_mean=gm)
        cidx, gidx = hga.route_ex(Q, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                                  layout=layout)
        O, lse = hga.attend_ex(Q, K, V, gidx, w.group, layout=layout, seq_len=w.T)
        cm2, gm2 = cm.clone(), gm.clone()
        step = hga.decode_step_ex(Q, K, V, cm2, gm2, w.T, w.chunk, w.group, w.k_chunk,
                                  w.k_group, layout=layout)
        torch.cuda.synchronize()
        return [cm, gm, cidx, gidx, O, lse, cm2, gm2, *step]

    got = run([w.T + 500, -7, w.T - 100])
    want = run([w.T, 0, w.T - 100])
    for i, (x, y) in enumerate(zip(got, want)):
        assert torch.equal(x, y), i
    assert (want[3][1] == -1).all()     # the empty sequence routes to nothing


def test_paged_cache_matches_ragged_dense():
    log("case paged")
    w, inp, seq_lens = _ragged_case(1)
    lens = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    dense = _run_ragged(w, inp, seq_lens, hga.Layout(seq_lens=lens), to_dev(inp.K, w.dtype),
                        to_dev(inp.V, w.dtype))
    kp, vp, table, n_pages = _pages(w, inp, seq_lens, 64)
    layout = hga.Layout(seq_lens=lens, block_table=table, page_tokens=64, n_pages=n_pages)
    paged = _run_ragged(w, inp, seq_lens, layout, kp, vp)
    for b, Tb in enumerate(seq_lens):       # same arithmetic in the same order: bit-identical
        nc, ng = -(-Tb // w.chunk), -(-Tb // w.group)
        assert torch.equal(paged["cm"][b, :, :nc], dense["cm"][b, :, :nc])
        assert torch.equal(paged["gm"][b, :, :ng], dense["gm"][b, :, :ng])
    for k in ("cidx", "gidx", "O", "lse"):
        assert torch.equal(paged[k], dense[k]), k
    from tests.gpu_runner import check_ragged
    check_ragged(w, inp, seq_lens, paged)
    # decode refresh: every sequence's newest key changes; refresh = rebuild
    for b, Tb in enumerate(seq_lens):
        pid = int(table[b, (Tb - 1) // 64])
        kp[pid, :, (Tb - 1) % 64] += 1.0
    hga.update_summaries_ex(kp, w.chunk, w.group, 1, paged["cm"], paged["gm"], layout=layout,
                            seq_len=w.T)
    cm2, gm2 = hga.build_summaries_ex(kp, w.chunk, w.group, layout=layout, seq_len=w.T)
    torch.cuda.synchronize()
    for b, Tb in enumerate(seq_lens):
        nc, ng = -(-Tb // w.chunk), -(-Tb // w.group)
        assert torch.equal(paged["cm"][b, :, :nc], cm2[b, :, :nc])
        assert torch.equal(paged["gm"][b, :, :ng], gm2[b, :, :ng])


def test_ragged_query_before_first_key():
    """A sequence shorter than Nq: the query at a negative position routes to
    nothing (-1 ids, O = 0, lse = -inf); the next sees only token 0."""
    log("case ragged-short")
    w = DECODE_64K.with_(B=2, Hq=4, Hkv=1, T=512, Nq=2, k_chunk=1, k_group=2, plants=0)
    inp = generate(w)
    lens = torch.tensor([512, 1], dtype=torch.int32, device="cuda")
    out = _run_ragged(w, inp, [512, 1], hga.Layout(seq_lens=lens), to_dev(inp.K, w.dtype),
                      to_dev(inp.V, w.dtype))
    assert (out["gidx"][1, :, 0] == -1).all() and (out["cidx"][1, :, 0] == -1).all()
    assert (out["O"][1, :, 0] == 0).all() and torch.isinf(out["lse"][1, :, 0]).all()
    assert (out["gidx"][1, :, 1, 0] == 0).all() and (out["gidx"][1, :, 1, 1:] == -1).all()
    O1 = out["O"][1, :, 1].float().cpu().numpy()
    assert np.abs(O1 - inp.V[1, 0, 0]).max() < 1e-2     # softmax over one token


def test_one_workspace_serves_calls_of_different_shapes():
    """Regression: a workspace reused across shapes. The first call's scores
    must never land where the second call's arrival counters live."""
    log("case workspace-reuse-across-shapes")
    w1, w2 = FUSED_ROUTE
    big = max(hga.route_workspace_bytes(hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D), w.chunk,
                                        w.group, w.k_chunk, w.k_group) for w in (w1, w2))
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for w in (w1, w2, w1):
        inp = generate(w)
        Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
        cm, gm = hga.build_summaries(K, w.chunk, w.group)
        cidx, gidx = hga.route(Q, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group, workspace=ws)
        O, lse = hga.attend(Q, K, V, gidx, w.group)
        torch.cuda.synchronize()
        check_workload(w, inp, dict(cm=cm, gm=gm, cidx=cidx, gidx=gidx, O=O, lse=lse))


@pytest.mark.parametrize("case", ["dense", "paged", "fallback-many-rows", "paged-crossing",
                                  "lean-crossing", "gpc16", "f32-d64"])
def test_route_fresh_equals_update_then_route(case):
    """hga_route_fresh_ex (refresh of the newest keys' chunks fused into
    routing) gives the summaries and routes of update-then-route, bit for bit,
    and those match the oracle on the new keys. The crossing cases put the
    newest keys of some sequences on both sides of a chunk boundary, in the
    one-workgroup-per-CU form and in the two-per-CU form (512 rows); gpc16 has
    16 groups per chunk, more than a workgroup has waves; f32-d64 refreshes
    fp32 keys of 64 dims (one load pass per group, as bf16 keys)."""
    log(f"case route-fresh-{case}")
    seq_lens, paged = None, case in ("paged", "paged-crossing")
    if case == "fallback-many-rows":
        w = DECODE_64K.with_(B=40, T=4096, k_chunk=2, k_group=4, plants=1)
    elif case == "lean-crossing":
        w = DECODE_64K.with_(B=8, T=4096, Nq=2, k_chunk=2, k_group=4, plants=1)
        seq_lens = [w.T if b % 2 == 0 else 15 * w.chunk + 1 for b in range(w.B)]
    elif case == "gpc16":
        w = DECODE_64K.with_(B=2, T=8192, group=16, k_chunk=4, k_group=16, plants=2)
    elif case == "f32-d64":
        w = DECODE_64K.with_(B=2, T=4096, D=64, k_chunk=3, k_group=12, plants=1, dtype="f32")
    else:
        w = DECODE_64K.with_(B=2, T=8192, Nq=2, k_chunk=4, k_group=8, plants=2)
        if case == "paged":
            seq_lens = [w.T, w.T - 100]
        elif case == "paged-crossing":
            seq_lens = [w.T, 31 * w.chunk + 1]
    inp = generate(w)
    Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
    layout, Kc, Vc = None, K, V
    if seq_lens is not None:
        lens = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
        if paged:
            kp, vp, table, n_pages = _pages(w, inp, seq_lens, 64)
            layout = hga.Layout(seq_lens=lens, block_table=table, page_tokens=64, n_pages=n_pages)
            Kc, Vc = kp, vp
        else:
            layout = hga.Layout(seq_lens=lens)
    cm, gm = hga.build_summaries_ex(Kc, w.chunk, w.group, layout=layout, seq_len=w.T)
    # the newest keys change after the summaries were built (a decode step appended them)
    if seq_lens is None:
        Kc[:, :, -w.Nq:] += 0.75
    else:
        for b, Tb in enumerate(seq_lens):
            for t in range(Tb - w.Nq, Tb):
                if paged:
                    Kc[int(table[b, t // 64]), :, t % 64] += 0.75
                else:
                    Kc[b, :, t] += 0.75
    cm_f, gm_f = cm.clone(), gm.clone()
    _, g_fresh = hga.route_fresh_ex(Q, Kc, cm_f, gm_f, w.T, w.chunk, w.group, w.k_chunk,
                                    w.k_group, layout=layout)
    cm_r, gm_r = cm.clone(), gm.clone()
    hga.update_summaries_ex(Kc, w.chunk, w.group, w.Nq, cm_r, gm_r, layout=layout, seq_len=w.T)
    _, g_ref = hga.route_ex(Q, cm_r, gm_r, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                            layout=layout)
    cm_b, gm_b = hga.build_summaries_ex(Kc, w.chunk, w.group, layout=layout, seq_len=w.T)
    torch.cuda.synchronize()
    assert torch.equal(g_fresh, g_ref)
    if seq_lens is None:
        assert torch.equal(cm_f, cm_r) and torch.equal(gm_f, gm_r)
        assert torch.equal(cm_f, cm_b) and torch.equal(gm_f, gm_b)
    else:
        for b, Tb in enumerate(seq_lens):
            nc, ng = -(-Tb // w.chunk), -(-Tb // w.group)
            assert torch.equal(cm_f[b, :, :nc], cm_r[b, :, :nc])
            assert torch.equal(gm_f[b, :, :ng], gm_r[b, :, :ng])
            assert torch.equal(cm_f[b, :, :nc], cm_b[b, :, :nc])
            assert torch.equal(gm_f[b, :, :ng], gm_b[b, :, :ng])
    if case in ("dense", "gpc16", "f32-d64"):   # and the oracle on the modified keys agrees
        from synth.inputs import Inputs
        inp2 = Inputs(w, inp.seed, inp.Q, Kc.float().cpu().numpy(), inp.V)
        cidx, gidx = hga.route(Q, cm_b, gm_b, w.T, w.chunk, w.group, w.k_chunk, w.k_group)
        O, lse = hga.attend(Q, Kc, Vc, g_fresh, w.group)
        torch.cuda.synchronize()
        check_workload(w, inp2, dict(cm=cm_f, gm=gm_f, cidx=cidx, gidx=g_fresh, O=O, lse=lse))


def _bump_newest(w, Kc, layout_info):
    """The newest keys of every sequence change after the summaries were built
    (a decode step appended them)."""
    if layout_info is None:
        Kc[:, :, -w.Nq:] += 0.75
    else:
        seq_lens, table, page_tokens = layout_info
        for b, Tb in enumerate(seq_lens):
            for t in range(Tb - w.Nq, Tb):
                Kc[int(table[b, t // page_tokens]), :, t % page_tokens] += 0.75


def _same_attention(O_a, lse_a, O_b, lse_b, dtype):
    """Two attention results over the same routed tokens whose fp32 partial
    sums were grouped differently: equal to fp32 rounding, so bf16 outputs
    differ by at most one bf16 step."""
    a, b = O_a.float(), O_b.float()
    d = (a - b).abs()
    if dtype == "bf16":
        lim = torch.maximum(a.abs(), b.abs()) * 2.0 ** -7 + 1e-6
    else:
        lim = torch.maximum(a.abs(), b.abs()) * 1e-5 + 1e-6
    assert bool((d <= lim).all()), f"O differs by up to {float(d.max()):.3g}"
    # rows without keys have lse = -inf on both sides
    assert torch.equal(torch.isneginf(lse_a), torch.isneginf(lse_b))
    fin = torch.isfinite(lse_a)
    if bool(fin.any()):
        assert float((lse_a[fin] - lse_b[fin]).abs().max()) <= 1e-4


def _zero_regions_are_zero():
    """Every workspace the binding keeps has its zero region back at zero."""
    Z = hga.WORKSPACE_ZERO_BYTES
    for key, buf in hga._ws.items():
        if key[1] in ("route", "attend", "decode", "staged"):   # not the staging pools
            assert int(buf[:Z].count_nonzero()) == 0, key


DECODE_CASES = {
    "bf16-b2-t8192-nq2": DECODE_64K.with_(B=2, T=8192, Nq=2, k_chunk=4, k_group=8, plants=2),
    "f32-b1-t4096": DECODE_64K.with_(B=1, T=4096, k_chunk=3, k_group=12, plants=1, dtype="f32"),
    "bf16-paged-ragged": DECODE_64K.with_(B=2, T=8192, Nq=2, k_chunk=4, k_group=8, plants=2),
    "bf16-fallback-many-rows": DECODE_64K.with_(B=40, T=4096, k_chunk=2, k_group=4, plants=1),
    "qwen3-b1-t65536": DECODE_64K,
    # one launch with both selection orders: the row at position 8191 ranks
    # chunks while the refreshed words arrive, the row at 8192 (chunk 32, after
    # the first refreshed chunk) waits for every word first
    "bf16-b2-t8193-nq2-across-chunk": DECODE_64K.with_(B=2, T=8193, Nq=2, k_chunk=4, k_group=8,
                                                       plants=2),
}


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_step_equals_fresh_route_then_attend(case):
    """hga_decode_step_ex (refresh + route + attend, one launch where the row
    route applies) gives the summaries and routes of route_fresh_ex bit for
    bit and the attention of attend_ex to fp32 rounding; on the dense case the
    whole step also matches the oracle on the modified keys."""
    w = DECODE_CASES[case]
    log(f"case decode-step-{case} {w.name} B={w.B} T={w.T} Nq={w.Nq}")
    inp = generate(w)
    Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
    layout, Kc, Vc, info = None, K, V, None
    if "paged" in case:
        seq_lens = [w.T, w.T - 100]
        kp, vp, table, n_pages = _pages(w, inp, seq_lens, 64)
        lens = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
        layout = hga.Layout(seq_lens=lens, block_table=table, page_tokens=64, n_pages=n_pages)
        Kc, Vc, info = kp, vp, (seq_lens, table, 64)
    if "across-chunk" in case:
        assert hga.decode_step_one_launch(hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D), w.dtype,
                                          w.chunk, w.group, w.k_chunk, w.k_group)
    cm, gm = hga.build_summaries_ex(Kc, w.chunk, w.group, layout=layout, seq_len=w.T)
    _bump_newest(w, Kc, info)
    cm_d, gm_d = cm.clone(), gm.clone()
    O_d, lse_d, c_d, g_d = hga.decode_step_ex(Q, Kc, Vc, cm_d, gm_d, w.T, w.chunk, w.group,
                                              w.k_chunk, w.k_group, layout=layout)
    cm_r, gm_r = cm.clone(), gm.clone()
    c_r, g_r = hga.route_fresh_ex(Q, Kc, cm_r, gm_r, w.T, w.chunk, w.group, w.k_chunk,
                                  w.k_group, layout=layout)
    O_r, lse_r = hga.attend_ex(Q, Kc, Vc, g_r, w.group, layout=layout, seq_len=w.T)
    torch.cuda.synchronize()
    assert torch.equal(g_d, g_r) and torch.equal(c_d, c_r)
    assert torch.equal(cm_d, cm_r) and torch.equal(gm_d, gm_r)
    _zero_regions_are_zero()
    _same_attention(O_d, lse_d, O_r, lse_r, w.dtype)
    # the step's own outputs against the oracle on the modified keys
    from synth.inputs import Inputs
    if layout is None:
        inp2 = Inputs(w, inp.seed, inp.Q, Kc.float().cpu().numpy(), inp.V)
        check_workload(w, inp2, dict(cm=cm_d, gm=gm_d, cidx=c_d, gidx=g_d, O=O_d, lse=lse_d))
    else:
        # the logical dense cache with the same bf16 update of each newest key
        Kd = torch.from_numpy(inp.K).to(torch.bfloat16)
        for b, Tb in enumerate(info[0]):
            Kd[b, :, Tb - w.Nq:Tb] += 0.75
        inp2 = Inputs(w, inp.seed, inp.Q, Kd.float().numpy(), inp.V)
        from tests.gpu_runner import check_ragged
        check_ragged(w, inp2, info[0], dict(cm=cm_d, gm=gm_d, cidx=c_d, gidx=g_d, O=O_d,
                                            lse=lse_d))


# More than 2048 items for one wave to select from (4094 middle chunks: 64 keys
# per lane), through every routing form: the row route, the refreshing row
# route, the one-launch decode step, and the MFMA prefill route's select
# kernel (16 queries per head).
WIDE = DECODE_64K.with_(name="wide-c16-g8-t65536", Hq=4, Hkv=1, chunk=16, group=8, k_chunk=64,
                        k_group=32, plants=4)


@pytest.mark.parametrize("Nq", [1, 16])
def test_select_over_4094_chunks(Nq):
    w = WIDE.with_(Nq=Nq)
    log(f"case {w.name} Nq={Nq}")
    shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
    inp = generate(w)
    out = run_hip(w, inp)
    check_workload(w, inp, out)
    Q, K, V = out["Q"], out["K"], out["V"]
    cm, gm = out["cm"].clone(), out["gm"].clone()
    c_f, g_f = hga.route_fresh_ex(Q, K, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group)
    torch.cuda.synchronize()
    assert torch.equal(c_f, out["cidx"]) and torch.equal(g_f, out["gidx"])
    if Nq == 1:
        assert hga.decode_step_one_launch(shape, w.dtype, w.chunk, w.group, w.k_chunk, w.k_group)
    cm2, gm2 = out["cm"].clone(), out["gm"].clone()
    O, lse, c_d, g_d = hga.decode_step_ex(Q, K, V, cm2, gm2, w.T, w.chunk, w.group, w.k_chunk,
                                          w.k_group, check=True)
    torch.cuda.synchronize()
    check_workload(w, inp, dict(cm=cm2, gm=gm2, cidx=c_d, gidx=g_d, O=O, lse=lse))
    assert torch.equal(c_d, out["cidx"]) and torch.equal(g_d, out["gidx"])


# The chunk level with one key slot per lane fewer than the group level: 1967
# middle chunks (31 keys per lane) against 2008 group candidates (32 keys per
# lane), so the chunk level ranks with 31 slots and the group level with 32,
# through the row route, the refreshing row route and the one-launch decode step.
NARROW_L1 = DECODE_64K.with_(name="l1-slot-fewer-c32-g8-t63000", Hq=4, Hkv=1, T=63000, chunk=32,
                             group=8, k_chunk=500, k_group=64, plants=4)


def test_chunk_level_one_slot_fewer():
    w = NARROW_L1
    log(f"case {w.name}")
    shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
    inp = generate(w)
    out = run_hip(w, inp)
    check_workload(w, inp, out)
    Q, K, V = out["Q"], out["K"], out["V"]
    cm, gm = out["cm"].clone(), out["gm"].clone()
    c_f, g_f = hga.route_fresh_ex(Q, K, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group)
    torch.cuda.synchronize()
    assert torch.equal(c_f, out["cidx"]) and torch.equal(g_f, out["gidx"])
    assert hga.decode_step_one_launch(shape, w.dtype, w.chunk, w.group, w.k_chunk, w.k_group)
    cm2, gm2 = out["cm"].clone(), out["gm"].clone()
    O, lse, c_d, g_d = hga.decode_step_ex(Q, K, V, cm2, gm2, w.T, w.chunk, w.group, w.k_chunk,
                                          w.k_group, check=True)
    torch.cuda.synchronize()
    check_workload(w, inp, dict(cm=cm2, gm=gm2, cidx=c_d, gidx=g_d, O=O, lse=lse))
    assert torch.equal(c_d, out["cidx"]) and torch.equal(g_d, out["gidx"])


def test_decode_step_status_word_is_sticky_until_reset():
    """A workspace whose status word says an earlier wait gave up: the next
    one-launch decode step reads no hand-off word and poisons every row (NaN
    O and lse, -1 ids) while still refreshing the summaries; the check reports
    HGA_ERR_TIMEOUT until the workspace is reset, after which the step is
    exact again. (The flag is set from the host: no kernel waits in vain.)"""
    w = DECODE_64K.with_(B=2, T=8192, k_chunk=4, k_group=8, plants=2)
    log("case decode-step-status-word")
    shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
    assert hga.decode_step_one_launch(shape, w.dtype, w.chunk, w.group, w.k_chunk, w.k_group)
    inp = generate(w)
    Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
    cm0, gm0 = hga.build_summaries(K, w.chunk, w.group)
    K[:, :, -1] += 0.75            # the newest key changed after the summaries were built
    nbytes = hga.decode_step_workspace_bytes(shape, w.chunk, w.group, w.k_chunk, w.k_group)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    Z = hga.WORKSPACE_ZERO_BYTES

    def step(check):
        cm, gm = cm0.clone(), gm0.clone()
        res = hga.decode_step_ex(Q, K, V, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                                 workspace=ws, check=check)
        torch.cuda.synchronize()
        return res, cm, gm

    (O, lse, c, g), cm, gm = step(True)
    ws[Z - 256:Z - 252] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device="cuda")
    (O2, lse2, c2, g2), cm2, gm2 = step(False)
    assert bool(torch.isnan(O2.float()).all()) and bool(torch.isnan(lse2).all())
    assert bool((g2 == -1).all()) and bool((c2 == -1).all())
    assert torch.equal(cm2, cm) and torch.equal(gm2, gm)
    with pytest.raises(hga.HGAError) as err:
        hga.workspace_check(ws)
    assert err.value.status == hga.ERR_TIMEOUT
    hga.workspace_reset(ws)
    hga.workspace_check(ws)
    assert int(ws[:Z].count_nonzero()) == 0
    (O3, lse3, c3, g3), _, _ = step(True)
    assert torch.equal(O3, O) and torch.equal(lse3, lse)
    assert torch.equal(c3, c) and torch.equal(g3, g)
    assert int(ws[:Z].count_nonzero()) == 0


def test_decode_step_one_launch_ragged_short_and_empty():
    """One-launch decode step over a ragged dense batch holding an empty
    sequence and one shorter than the number of new queries (its first query
    sits before its first key): routes and summaries equal route_fresh_ex's bit
    for bit, attention equals attend_ex's to fp32 rounding, rows without keys
    give O = 0 and lse = -inf, and the workspace's zero region is left zero."""
    w = DECODE_64K.with_(B=3, Hq=8, Hkv=2, T=4096, Nq=3, k_chunk=4, k_group=8, plants=1)
    seq_lens = [w.T, 2, 0]
    log(f"case decode-step-ragged-short-empty seq_lens={seq_lens}")
    shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
    assert hga.decode_step_one_launch(shape, w.dtype, w.chunk, w.group, w.k_chunk, w.k_group)
    inp = generate(w)
    Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
    lens = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    layout = hga.Layout(seq_lens=lens)
    cm, gm = hga.build_summaries_ex(K, w.chunk, w.group, layout=layout, seq_len=w.T)
    for b, Tb in enumerate(seq_lens):   # the newest keys changed after the build
        K[b, :, max(0, Tb - w.Nq):Tb] += 0.75
    cm_d, gm_d = cm.clone(), gm.clone()
    O_d, lse_d, c_d, g_d = hga.decode_step_ex(Q, K, V, cm_d, gm_d, w.T, w.chunk, w.group,
                                              w.k_chunk, w.k_group, layout=layout)
    cm_r, gm_r = cm.clone(), gm.clone()
    c_r, g_r = hga.route_fresh_ex(Q, K, cm_r, gm_r, w.T, w.chunk, w.group, w.k_chunk,
                                  w.k_group, layout=layout)
    O_r, lse_r = hga.attend_ex(Q, K, V, g_r, w.group, layout=layout, seq_len=w.T)
    torch.cuda.synchronize()
    assert torch.equal(g_d, g_r) and torch.equal(c_d, c_r)
    assert torch.equal(cm_d, cm_r) and torch.equal(gm_d, gm_r)
    _same_attention(O_d, lse_d, O_r, lse_r, w.dtype)
    # rows with no key at or before their position: the empty sequence, and
    # the short sequence's first query (position 2 - 3 + 0 < 0)
    for b, i in [(2, 0), (2, 1), (2, 2), (1, 0)]:
        assert bool((g_d[b, :, i] == -1).all())
        assert bool((O_d[b, :, i].float() == 0).all())
        assert bool(torch.isneginf(lse_d[b, :, i]).all())
    assert bool((g_d[1, :, 1:, 0] >= 0).all())   # the short sequence's later queries see keys
    _zero_regions_are_zero()


def test_decode_step_back_to_back_leaves_counters_zero():
    """Successive one-launch decode steps on one workspace (each step's queries
    differ; only its zero region is zero at the start) each match the two-call
    result, and leave the zero region (counters and score words) at zero."""
    log("case decode-step back-to-back")
    # two attention workgroups per row, so the arrival counters are used too
    w = DECODE_64K.with_(B=2, T=16384, k_chunk=8, k_group=64, plants=2)
    inp = generate(w)
    Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
    cm, gm = hga.build_summaries(K, w.chunk, w.group)
    shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
    nbytes = hga.decode_step_workspace_bytes(shape, w.chunk, w.group, w.k_chunk, w.k_group)
    # a workspace that an earlier call of another shape left dirty past its counters
    ws = torch.full((nbytes + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    Z = hga.WORKSPACE_ZERO_BYTES
    ws[:Z] = 0
    for step in range(4):
        Qs = (Q.float() * (1.0 + 0.25 * step)).to(Q.dtype) if step % 2 else Q.flip(1).contiguous()
        O_d, lse_d, _, g_d = hga.decode_step_ex(Qs, K, V, cm, gm, w.T, w.chunk, w.group,
                                                w.k_chunk, w.k_group, workspace=ws)
        # the two-call form on the same workspace: it must leave the zero region alone
        _, g_r = hga.route_fresh_ex(Qs, K, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                                    workspace=ws)
        O_r, lse_r = hga.attend(Qs, K, V, g_r, w.group, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(g_d, g_r), step
        _same_attention(O_d, lse_d, O_r, lse_r, w.dtype)
        assert int(ws[:Z].count_nonzero()) == 0


def test_prefill_ragged_with_queries_before_the_first_key():
    """Prefill (MFMA route) over a ragged batch: the shortest sequence holds
    fewer keys than there are new queries, so its first queries route to
    nothing; every other query matches the oracle run on its own sequence."""
    log("case prefill-ragged")
    w = Workload("prefill-ragged", 3, 8, 2, 128, 2048, 40, 128, 32, 3, 6, 1e4, "bf16", 0)
    seq_lens = [2048, 1000, 25]
    inp = generate(w)
    lens = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    out = _run_ragged(w, inp, seq_lens, hga.Layout(seq_lens=lens), to_dev(inp.K, w.dtype),
                      to_dev(inp.V, w.dtype))
    from synth.inputs import Inputs
    from tests.gpu_runner import check_ragged
    check_ragged(w.with_(B=2), inp, seq_lens[:2], {k: v[:2] for k, v in out.items()})
    Tb, short = seq_lens[2], w.Nq - seq_lens[2]          # queries 0..short-1 sit before key 0
    assert (out["gidx"][2, :, :short] == -1).all() and (out["cidx"][2, :, :short] == -1).all()
    assert (out["O"][2, :, :short] == 0).all() and torch.isinf(out["lse"][2, :, :short]).all()
    wb = w.with_(B=1, T=Tb, Nq=Tb)
    sub = Inputs(wb, inp.seed, inp.Q[2:3, :, short:], inp.K[2:3, :, :Tb], inp.V[2:3, :, :Tb])
    ob = dict(cm=out["cm"][2:3, :, :wb.n_chunks], gm=out["gm"][2:3, :, :wb.n_groups],
              cidx=out["cidx"][2:3, :, short:], gidx=out["gidx"][2:3, :, short:],
              O=out["O"][2:3, :, short:], lse=out["lse"][2:3, :, short:])
    check_workload(wb, sub, ob)


@pytest.mark.parametrize("paged", [False, True], ids=["dense", "paged"])
def test_prefill_tiles_ragged(paged):
    """Tile attention (128-row tiles over the union of routed groups) on a
    ragged batch, dense or paged: the shortest sequence holds fewer keys than
    there are new queries, so a tile starts with rows that route to nothing;
    every other query matches the oracle run on its own sequence."""
    log(f"case prefill-tiles-ragged paged={paged}")
    w = Workload("prefill-tiles-ragged", 3, 4, 2, 128, 2048, 150, 128, 32, 3, 6, 1e4, "bf16", 0)
    seq_lens = [2048, 1000, 100]
    inp = generate(w)
    lens = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    if paged:
        kp, vp, table, n_pages = _pages(w, inp, seq_lens, 64)
        layout = hga.Layout(seq_lens=lens, block_table=table, page_tokens=64, n_pages=n_pages)
        out = _run_ragged(w, inp, seq_lens, layout, kp, vp)
    else:
        out = _run_ragged(w, inp, seq_lens, hga.Layout(seq_lens=lens), to_dev(inp.K, w.dtype),
                          to_dev(inp.V, w.dtype))
    from synth.inputs import Inputs
    from tests.gpu_runner import check_ragged
    check_ragged(w.with_(B=2), inp, seq_lens[:2], {k: v[:2] for k, v in out.items()})
    Tb, short = seq_lens[2], w.Nq - seq_lens[2]          # queries 0..short-1 sit before key 0
    assert (out["gidx"][2, :, :short] == -1).all()
    assert (out["O"][2, :, :short] == 0).all() and torch.isinf(out["lse"][2, :, :short]).all()
    wb = w.with_(B=1, T=Tb, Nq=Tb)
    sub = Inputs(wb, inp.seed, inp.Q[2:3, :, short:], inp.K[2:3, :, :Tb], inp.V[2:3, :, :Tb])
    ob = dict(cm=out["cm"][2:3, :, :wb.n_chunks], gm=out["gm"][2:3, :, :wb.n_groups],
              cidx=out["cidx"][2:3, :, short:], gidx=out["gidx"][2:3, :, short:],
              O=out["O"][2:3, :, short:], lse=out["lse"][2:3, :, short:])
    check_workload(wb, sub, ob)


@pytest.mark.parametrize("case", ["device-bf16", "pinned-bf16-overlap", "pinned-f32-padding"])
def test_attend_staged_equals_attend(case):
    """Staged attention (each (sequence, KV head)'s distinct routed groups
    copied once into a device pool) gives attend's results bit for bit, with
    device or pinned host K/V, overlapping routes across the heads of a KV
    head, and -1 padding."""
    log(f"case attend-staged-{case}")
    if case == "device-bf16":
        w = DECODE_64K.with_(B=2, T=8192, Nq=2, k_chunk=4, k_group=8, plants=2)
    elif case == "pinned-bf16-overlap":       # many groups per row: heads overlap
        w = DECODE_64K.with_(B=3, Hq=16, Hkv=2, T=4096, Nq=3, k_chunk=12, k_group=96, plants=0)
    else:
        w = Workload("staged-f32", 2, 4, 2, 64, 1000, 5, 64, 16, 2, 20, 1e4, "f32", 0)
    inp = generate(w)
    out = run_hip(w, inp)
    K, V = out["K"], out["V"]
    if case != "device-bf16":
        from tests.gpu_runner import to_pinned
        K, V = to_pinned(inp.K, w.dtype), to_pinned(inp.V, w.dtype)
    O_d, lse_d = hga.attend(out["Q"], K, V, out["gidx"], w.group)
    O_s, lse_s = hga.attend_staged(out["Q"], K, V, out["gidx"], w.group)
    torch.cuda.synchronize()
    assert torch.equal(O_s, O_d) and torch.equal(lse_s, lse_d)
    assert torch.equal(O_s, out["O"])
    if case == "pinned-f32-padding":         # the routing pads with -1 here
        assert (out["gidx"] == -1).any()


def test_attend_staged_host_tier_b4_t262144():
    """The host-memory tier workload through staged attention equals the
    direct reads of pinned host K/V, and moves about half the bytes."""
    w = HOST_TIER
    log(f"case attend-staged-{w.name}")
    inp = generate(w)
    out = run_hip(w, inp)          # direct: every row reads its groups from host memory
    O_s, lse_s = hga.attend_staged(out["Q"], out["K"], out["V"], out["gidx"], w.group)
    torch.cuda.synchronize()
    assert torch.equal(O_s, out["O"]) and torch.equal(lse_s, out["lse"])
    g = out["gidx"].cpu().numpy()
    r = w.Hq // w.Hkv
    distinct = sum(len(np.unique(g[b, kv * r:(kv + 1) * r][g[b, kv * r:(kv + 1) * r] >= 0]))
                   for b in range(w.B) for kv in range(w.Hkv))
    assert distinct < 0.75 * int((g >= 0).sum())
    # the benchmark's host-tier step routes with the refresh reading K from
    # host memory: same summaries and routes, bit for bit
    cm_f, gm_f = out["cm"].clone(), out["gm"].clone()
    c_f, g_f = hga.route_fresh_ex(out["Q"], out["K"], cm_f, gm_f, w.T, w.chunk, w.group,
                                  w.k_chunk, w.k_group)
    torch.cuda.synchronize()
    assert torch.equal(cm_f, out["cm"]) and torch.equal(gm_f, out["gm"])
    assert torch.equal(g_f, out["gidx"]) and torch.equal(c_f, out["cidx"])

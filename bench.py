#!/usr/bin/env python3
"""HGA routed-attention decode benchmark on one MI355X.

One step = one decode step of one attention layer over the whole batch, the
full hot path in one call (hga_decode_step_ex): refresh the summaries of the
chunks holding the newest keys, route with them, and attend exactly over the
routed tokens (one launch for small batches). Inputs are synthetic, seeded,
already resident in HBM when timing starts. Caches are kept cold by rotating over enough copies
of K/V/summaries that the routed working sets of one rotation exceed the
256 MB Infinity Cache. Steps replay HIP graphs (one per copy) unless --no-graph.

Prints one JSON line (metric, value in decode tokens/s, roofline of the
step's dominant kernel, of the attention kernel alone and of the whole step,
CPU-oracle baseline, per-kernel times, latency percentiles).

    python bench.py [--steps K] [--warmup W] [--workload NAME]
    python bench.py --only decode|attend|route|route_fresh|update|copy   # short runs for rocprofv3
    HGA_LIB=hierarchical_sparse_attention_summaries_amd/libhga_phases.so python bench.py --phases
        # per-phase clock stamps of the one-launch decode step (phase-stamp build)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-attn decode tokens/s + achieved HBM GB/s at 64K ctx, 1 MI355X"
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20
SECONDARY = "qwen3-30b-a3b-decode-b16-t65536"   # the 64K point of the batch-16 context sweep
HOST_TIER = "qwen3-30b-a3b-host-tier-b4-t262144"  # full K/V in pinned host memory
PREFILL = "qwen3-30b-a3b-prefill-nq4096-t65536"     # 4096 new tokens against a 64K cache
PEAK_MFMA_BF16_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3-30b-a3b-decode-b1-t65536")
    ap.add_argument("--sets", type=int, default=0, help="K/V copies rotated per step (0 = auto)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["decode", "attend", "route", "route_fresh", "update", "step",
                                       "build", "copy"])
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the batch-16 64K-context point of the context sweep")
    ap.add_argument("--no-host-tier", action="store_true",
                    help="skip the 256K-context batch-4 run with K/V in pinned host memory")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 4096-query prefill step against a 64K cache (MFMA scoring)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the batch-16 context sweep below 64K (4096..32768 tokens)")
    ap.add_argument("--phases", action="store_true",
                    help="per-phase stamps of the one-launch decode step (needs the phase-stamp "
                         "build of the library, loaded through HGA_LIB)")
    return ap.parse_args()


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "hierarchical_sparse_attention_summaries_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Sources each profiled kernel is built from: a stored counter reading is used
# only while they hash as they did when it was taken.
KERNEL_SOURCES = {
    "attend": ["attend.hip", "hga_attend_body.h", "hga_device.h", "hga_internal.h"],
    "decode_step": ["decode.hip", "hga_attend_body.h", "hga_route_row_launch.h",
                    "hga_route_row_body.h", "hga_device.h", "hga_internal.h", "hga_select.h",
                    "hga_summary.h"],
    "summaries": ["summaries.hip", "hga_summary.h", "hga_device.h", "hga_internal.h"],
}


def cache_read_rate(torch, dev, reps=50):
    """What the Infinity Cache delivers to a plain streaming read: the summary
    build (every key read once, small writes) over a 128 MiB bf16 key cache,
    warm: past the 32 MB of L2, within the 256 MB cache. GB/s of keys read."""
    import hierarchical_sparse_attention_summaries_amd as hga

    K = torch.randn((1, 4, 131072, 128), device=dev).to(torch.bfloat16)
    cm, gm = hga.build_summaries(K, 256, 32)
    for _ in range(5):
        hga.build_summaries(K, 256, 32, chunk_mean=cm, group_mean=gm)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    e0.record()
    for _ in range(reps):
        hga.build_summaries(K, 256, 32, chunk_mean=cm, group_mean=gm)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3
    return {"kernel": "hga_summaries", "bytes_read": K.numel() * 2,
            "read_gbs": round(K.numel() * 2 * reps / sec / 1e9, 1)}


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"hga_{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None, None
    m = re.search(r"^traffic_json: (\{.*\})\s*$", open(path).read(), flags=re.M)
    if not m:
        return None, None
    d = json.loads(m.group(1))
    if d.get("src_hash") != kernel_source_hash(KERNEL_SOURCES[kernel]):
        return None, d
    fetch = d["fetch_kib"] * 1024 * d["fetch_scale"]
    write = d["write_kib"] * 1024 * d["write_scale"]
    return fetch + write, d


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: HGA routed attention here runs on a single "
              "MI355X (multi-GPU sharding is a design note, not built). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import ALL

    w = ALL[args.workload]
    # The CPU oracle runs first, in forked worker processes, before anything
    # touches the GPU (the workers inherit no GPU state and are gone before it
    # is initialised).
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = cpu_baselines(w, args.cpu_seconds)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.phases:
        print(json.dumps(decode_phases(w, max(10, args.steps))))
        return

    if args.only == "copy":
        # Plain copy of known size, to scale rocprofv3 FETCH_SIZE / WRITE_SIZE.
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read": n, "bytes_written": n, "launches": args.steps}))
        return

    out = measure(w, args, primary=True)
    out["cpu_baseline"] = cpu
    out["run_conditions"] = run_conditions(torch)
    if not args.no_host_tier and w.name != HOST_TIER:
        h_args = argparse.Namespace(**vars(args))
        h_args.steps, h_args.warmup = 10, 2
        ht = measure(ALL[HOST_TIER], h_args, primary=False)
        out["host_tier"] = {k: ht[k] for k in ("config", "value", "unit", "ms_per_step", "steps",
                                               "kernels_us", "host_tier")}
        # HBM held against context length with K/V in host memory: the same
        # workload at 64K, 128K and 256K (budget held at ~3%)
        points = []
        for T in (65536, 131072):
            wt = ALL[HOST_TIER].with_(name=f"qwen3-30b-a3b-host-tier-b4-t{T}", T=T,
                                      k_chunk=T // 2048, k_group=T // 1024)
            s_args = argparse.Namespace(**vars(h_args))
            s_args.steps, s_args.warmup = 5, 1
            points.append(measure(wt, s_args, primary=False))
        points.append(ht)
        out["host_tier"]["memory_slope"] = host_memory_slope(points)
    if not args.no_prefill and w.name != PREFILL:
        p_args = argparse.Namespace(**vars(args))
        p_args.steps, p_args.warmup = 5, 2
        pf = measure(ALL[PREFILL], p_args, primary=False)
        out["prefill"] = {k: pf[k] for k in ("config", "value", "unit", "ms_per_step", "steps",
                                             "kernels_us", "roofline", "roofline_attend",
                                             "roofline_step", "roofline_build", "mfma")}
    if not args.no_sweep:
        # the batch-16 context sweep; its 64K point is the secondary run below
        from synth import SWEEP
        s_args = argparse.Namespace(**vars(args))
        s_args.steps, s_args.warmup = 40, 10
        out["sweep"] = []
        for T in sorted(SWEEP):
            ws = SWEEP[T]
            if ws.name in (w.name, SECONDARY):
                continue
            r = measure(ws, s_args, primary=False)
            out["sweep"].append({"seq_len": T, "value": r["value"], "unit": r["unit"],
                                 "ms_per_step": r["ms_per_step"], "steps": r["steps"],
                                 "attend_gbs": r["roofline_attend"]["achieved"],
                                 "attend_frac": r["roofline_attend"]["frac"],
                                 "step_gbs": r["roofline_step"]["achieved"],
                                 "kernels_us": r["kernels_us"]})
    if not args.no_secondary:
        w2 = ALL[SECONDARY]
        if w2.name != w.name:
            sec_args = argparse.Namespace(**vars(args))
            sec_args.steps, sec_args.warmup = max(50, args.steps // 4), max(5, args.warmup // 4)
            sec = measure(w2, sec_args, primary=False)
            out["secondary"] = {k: sec[k] for k in ("config", "value", "unit", "ms_per_step",
                                                    "steps", "hbm_gbs_step", "roofline",
                                                    "roofline_attend", "roofline_step",
                                                    "roofline_build", "warm_cache",
                                                    "kernels_us", "latency_us")}
    print(json.dumps(out))


def measure(w, args, primary: bool):
    import numpy as np
    import torch

    import hierarchical_sparse_attention_summaries_amd as hga
    from synth import generate

    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    esize = 2 if w.dtype == "bf16" else 4
    t_gen = time.time()
    inp = generate(w, seed=0)
    t_gen = time.time() - t_gen

    Q = torch.from_numpy(inp.Q).to(dev, tdt)
    if w.host_kv:   # full K/V in pinned host memory; summaries, Q, O in HBM
        K0 = torch.from_numpy(inp.K).to(tdt).pin_memory()
        V0 = torch.from_numpy(inp.V).to(tdt).pin_memory()
    else:
        K0 = torch.from_numpy(inp.K).to(dev, tdt)
        V0 = torch.from_numpy(inp.V).to(dev, tdt)
    cm0, gm0 = hga.build_summaries(K0, w.chunk, w.group)
    cidx0, gidx0 = hga.route(Q, cm0, gm0, w.T, w.chunk, w.group, w.k_chunk, w.k_group)
    torch.cuda.synchronize()

    # Algorithmic bytes (what the method must move).
    # The attention kernel alone: every row's routed K/V tokens, Q, O, lse, ids.
    g = gidx0.cpu().numpy()
    c = cidx0.cpu().numpy()
    r = w.Hq // w.Hkv
    rows = w.B * w.Hq * w.Nq
    gpc = w.chunk // w.group

    # tokens of group g usable by the query at position p (j <= p)
    pos = (w.T - w.Nq + np.arange(w.Nq)).reshape(1, 1, w.Nq, 1)
    ntok = np.clip(np.minimum(g * w.group + w.group, pos + 1) - g * w.group, 0, None)
    ntok = np.where(g >= 0, ntok, 0)
    routed_tokens = int(ntok.sum())
    union_tokens = 0      # K/V tokens routed to any query of a (sequence, KV head)
    union_cand = 0        # candidate group summaries read by any query of a (sequence, KV head)
    for b in range(w.B):
        for kv in range(w.Hkv):
            gs = g[b, kv * r:(kv + 1) * r].reshape(-1)
            ns = ntok[b, kv * r:(kv + 1) * r].reshape(-1)
            keep = gs >= 0
            if keep.any():   # a group's usable tokens: its largest count over the queries
                order = np.lexsort((-ns[keep], gs[keep]))
                gk, nk = gs[keep][order], ns[keep][order]
                first = np.ones(len(gk), dtype=bool)
                first[1:] = gk[1:] != gk[:-1]
                union_tokens += int(nk[first].sum())
            cs = np.unique(c[b, kv * r:(kv + 1) * r].reshape(-1))
            cs = cs[cs >= 0]
            cand = (cs[:, None] * gpc + np.arange(gpc)[None, :]).reshape(-1)
            union_cand += int((cand < w.n_groups).sum())
    # Attention's algorithmic HBM bytes take each KV head's routed K/V once (the
    # union over its queries); with many queries per head (prefill) most
    # gathers then hit in cache, and the per-row gathers are reported apart.
    attend_bytes = union_tokens * w.D * 2 * esize + rows * (2 * w.D * esize + 4 * w.k_group + 4)
    gather_bytes = routed_tokens * w.D * 2 * esize
    # Many queries per head (bf16, D 128, G 32, <= 2048 groups, >= 128 queries):
    # the attention runs in tiles of 128 rows of one head over the union of
    # their routed groups, on MFMA. Its bytes are each tile's union; its
    # executed MFMA work counts, for every 16-row wave, every group any of
    # its rows routed: 16 rows x 32 tokens x D for S^T, twice that for the
    # hi + lo products of O^T, 2 flops each.
    tiles = None
    if (w.dtype == "bf16" and w.D == 128 and w.group == 32 and w.n_groups <= 2048
            and w.Nq >= 128):
        n_union = n_wave_groups = n_tiles = 0
        for b in range(w.B):
            for h in range(w.Hq):
                for i0 in range(0, w.Nq, 128):
                    blk = g[b, h, i0:i0 + 128]
                    n_union += len(np.unique(blk[blk >= 0]))
                    n_tiles += 1
                    for w0 in range(0, blk.shape[0], 16):
                        wb = blk[w0:w0 + 16]
                        n_wave_groups += len(np.unique(wb[wb >= 0]))
        tiles = {"tiles": n_tiles, "union_groups_per_tile": round(n_union / n_tiles, 1),
                 "bytes": n_union * w.group * w.D * 2 * esize
                 + rows * (2 * w.D * esize + 4 * w.k_group + 4),
                 "executed_flops": n_wave_groups * 16 * w.group * w.D * 2 * 3,
                 "alg_flops": routed_tokens * w.D * 4}
    # One decode step: Q, all chunk summaries, the candidate groups' summaries,
    # the routed K/V (union per KV head), O, lse and ids, plus the refresh of the
    # chunks holding the newest keys (their keys read, their summaries written).
    c_first = (w.T - w.Nq) // w.chunk
    n_upd = w.n_chunks - c_first
    upd_tokens = w.T - c_first * w.chunk
    update_bytes = w.B * w.Hkv * (upd_tokens * w.D * esize + n_upd * (1 + gpc) * w.D * 4)
    step_bytes = (rows * w.D * esize + w.B * w.Hkv * w.n_chunks * w.D * 4 + union_cand * w.D * 4
                  + union_tokens * w.D * 2 * esize + rows * (w.D * esize + 4 + 4 * w.k_group)
                  + update_bytes)
    route_bytes = step_bytes - attend_bytes

    # Cold-cache rotation: copies at distinct addresses so that one rotation's
    # routed working sets exceed the Infinity Cache.
    per_set = attend_bytes + route_bytes
    S = args.sets or max(2, min(64, -(-2 * MALL_BYTES // per_set)))
    if w.host_kv:
        S = 1   # host memory is not kept in the GPU caches between steps
    sets = []
    for s in range(S):
        K = K0 if s == 0 else K0.clone()
        V = V0 if s == 0 else V0.clone()
        cm = cm0 if s == 0 else cm0.clone()
        gm = gm0 if s == 0 else gm0.clone()
        sets.append((K, V, cm, gm))
    shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
    ws_r = torch.zeros(hga.route_workspace_bytes(shape, w.chunk, w.group, w.k_chunk, w.k_group),
                       dtype=torch.uint8, device=dev)
    ws_a = torch.zeros(hga.attend_workspace_bytes(shape, w.group, w.k_group), dtype=torch.uint8,
                       device=dev)
    ws_d = torch.zeros(hga.decode_step_workspace_bytes(shape, w.chunk, w.group, w.k_chunk,
                                                       w.k_group), dtype=torch.uint8, device=dev)
    gidx = torch.empty_like(gidx0)
    O = torch.empty_like(Q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)

    def k_build(s):
        # step 1 in full (once per prefill; not part of a decode step)
        K, V, cm, gm = sets[s]
        hga.build_summaries(K, w.chunk, w.group, cm, gm)

    def k_update(s):
        K, V, cm, gm = sets[s]
        hga.update_summaries(K, w.chunk, w.group, w.T - w.Nq, w.T, cm, gm)

    def k_route(s):
        K, V, cm, gm = sets[s]
        hga.route(Q, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group, want_chunks=False,
                  group_idx=gidx, workspace=ws_r)

    def k_route_fresh(s):
        # steps 1-2 of a decode step: refresh the newest keys' summaries, route
        K, V, cm, gm = sets[s]
        hga.route_fresh_ex(Q, K, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                           want_chunks=False, group_idx=gidx, workspace=ws_r)

    def k_attend(s):
        K, V, cm, gm = sets[s]
        hga.attend(Q, K, V, gidx, w.group, out=O, lse=lse, workspace=ws_a)

    def k_decode(s):
        # the whole decode step: refresh, route, attend
        K, V, cm, gm = sets[s]
        hga.decode_step_ex(Q, K, V, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                           want_chunks=False, group_idx=gidx, out=O, lse=lse, workspace=ws_d)

    step = k_decode
    decode_one_launch = hga.decode_step_one_launch(shape, w.dtype, w.chunk, w.group, w.k_chunk,
                                                   w.k_group)
    if w.host_kv:
        # K/V in host memory: route (refreshing from host K), then copy each
        # (sequence, KV head)'s distinct routed groups into a device pool once
        # and attend from it
        pages, st_bytes = hga.attend_staged_sizes(shape, w.group, w.k_group)
        ws_st = torch.zeros(st_bytes, dtype=torch.uint8, device=dev)
        pools = tuple(torch.empty(pages * w.group * w.D, dtype=tdt, device=dev) for _ in range(2))

        def k_attend_staged(s):
            K, V, cm, gm = sets[s]
            hga.attend_staged(Q, K, V, gidx, w.group, out=O, lse=lse, pools=pools,
                              workspace=ws_st)

        def k_decode(s):
            k_route_fresh(s)
            k_attend_staged(s)

        step = k_decode
        decode_one_launch = False

    if args.only:
        fn = {"attend": k_attend, "route": k_route, "update": k_update, "step": step,
              "route_fresh": k_route_fresh, "decode": k_decode, "build": k_build}[args.only]
        k_route(0)
        for k in range(args.warmup + args.steps):
            fn(k % S)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "workload": w.name, "launches": args.warmup + args.steps,
                          "sets": S, "attend_alg_bytes": attend_bytes}))
        sys.exit(0)

    # correctness guard: the timed path reproduces the reference run's routing
    # and the standalone attention's output
    step(0)
    torch.cuda.synchronize()
    assert torch.equal(gidx, gidx0), "routing changed between runs"
    O_step = O.clone()
    k_attend(0)
    torch.cuda.synchronize()
    assert float((O_step.float() - O.float()).abs().max()) <= 2e-2, "decode step != attend"

    use_graph = not args.no_graph

    def capture(n, sets_used):
        """One graph of exactly n steps, rotating over the first sets_used copies."""
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for k in range(n):
                step(k % sets_used)
        return gr

    singles, graphs = [], {}
    if use_graph:
        for s in range(S):
            step(s)
        torch.cuda.synchronize()
        for s in range(S):       # single steps, for the latency percentiles
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(s)
            singles.append(gr)
        # The warm-up and the timed steps each replay one graph that holds
        # exactly that many steps (cold: rotating over the S copies; warm: one
        # copy, so the routed working set stays in the Infinity Cache), so that
        # no per-replay launch cost is spread over a few steps.
        for name, n, sets_used in (("warmup", args.warmup, S), ("cold", args.steps, S),
                                   ("warm", args.steps, 1)):
            if n > 0:
                graphs[name] = capture(n, sets_used)
        torch.cuda.synchronize()
    graphs_keep = (singles, graphs)

    def run(k):
        if use_graph:
            singles[k % S].replay()
        else:
            step(k % S)

    def run_steps(n, kind="cold"):
        """Exactly n steps, starting at copy 0 (kind "warm": copy 0 only)."""
        if n <= 0:
            return
        if use_graph:
            graphs[kind].replay()
            return
        for k in range(n):
            step(0 if kind == "warm" else k % S)

    def busy_gpu():
        # Keep the GPU busy while the host enqueues, so that event pairs time
        # the kernels and not the host's launch latency.
        try:
            torch.cuda._sleep(20_000_000)
        except Exception:
            a = torch.randn(4096, 4096, device=dev)
            for _ in range(20):
                a = a @ a
                a /= a.norm()

    # ---------------- timed region: exactly `steps` steps
    run_steps(args.warmup, "warmup")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = w.B * w.Nq / ((t1 - t0) / args.steps)

    # ---------------- the same steps with warm caches (one K/V copy, so the
    # routed working set stays in the Infinity Cache), beside the cold figure
    run_steps(args.steps, "warm")
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    run_steps(args.steps, "warm")
    torch.cuda.synchronize()
    tw1 = time.perf_counter()
    warm = {"ms_per_step": round((tw1 - tw0) * 1e3 / args.steps, 5),
            "value": round(w.B * w.Nq / ((tw1 - tw0) / args.steps), 1), "unit": "tokens/s",
            "steps": args.steps, "cache": "warm (one K/V copy reused every step)"}

    # ---------------- per-step latency percentiles (events between single-step replays)
    n_lat = max(50, min(args.steps, 400))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_lat + 1)]
    busy_gpu()
    evs[0].record()
    for k in range(n_lat):
        run(k)
        evs[k + 1].record()
    torch.cuda.synchronize()
    lat = sorted(evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(n_lat))

    def pct(a, q):
        return a[min(len(a) - 1, int(round(q * (len(a) - 1))))]

    # ---------------- per-kernel durations: HIP events on the stream the
    # kernels run on (torch's current stream) around n back-to-back eager
    # launches of one kernel (rotating over the copies), the GPU kept busy
    # while the host enqueues; average = elapsed / n.
    n_k = max(50, min(args.steps, 400))
    names = ["decode_step", "route_fresh", "attend", "update", "route"]   # the step is the first
    fns = [k_decode, k_route_fresh, k_attend, k_update, k_route]
    if not w.host_kv:   # a full build from host memory would take the link for seconds
        names.append("build")
        fns.append(k_build)
    if w.host_kv:
        names.append("attend_staged")
        fns.append(k_attend_staged)
    kern_us = {}
    for nm, fn in zip(names, fns):
        reps = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            busy_gpu()
            e0.record()
            for k in range(n_k):
                fn(k % S)
            e1.record()
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) * 1e3 / n_k)
        kern_us[nm] = {"avg": statistics.median(reps), "launches": 3 * n_k}
    attend_us = kern_us["attend"]["avg"]
    decode_us = kern_us["decode_step"]["avg"]

    quality = None
    if primary and not w.host_kv and w.Nq == 1:
        quality = quality_proxy(hga, torch, w, Q, sets[0][0], sets[0][1], gidx0)
    host = None
    if w.host_kv:
        kv_bytes = 2 * K0.numel() * esize
        hbm = sum(t.numel() * t.element_size()
                  for t in (Q, cm0, gm0, O, lse, gidx0, ws_d, ws_st, *pools))
        # staged: each (sequence, KV head)'s distinct routed groups cross the
        # host link once; direct: every row's groups do
        fetched = union_tokens * w.D * 2 * esize
        direct = gather_bytes
        host = {"kv_bytes_in_host_memory": kv_bytes, "hbm_bytes_resident": hbm,
                "fetched_bytes_per_token": fetched // (w.B * w.Nq),
                "host_link_gbs": round(fetched / (kern_us["attend_staged"]["avg"] * 1e-6) / 1e9, 2),
                "direct_fetched_bytes_per_token": direct // (w.B * w.Nq),
                "direct_attend_us": round(kern_us["attend"]["avg"], 1),
                "direct_host_link_gbs": round(direct / (kern_us["attend"]["avg"] * 1e-6) / 1e9, 2)}

    def roof(kernel, nbytes, us):
        traffic, _ = stored_traffic(kernel, w.name)
        achieved = nbytes / (us * 1e-6) / 1e9
        # HBM bytes the counters saw per launch, over the same launch time
        counter_gbs = round(traffic / (us * 1e-6) / 1e9, 1) if traffic else None
        return {"kernel": f"hga_{kernel}", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic, "traffic_gbs": counter_gbs,
                "traffic_over_alg": round(traffic / nbytes, 4) if traffic else None,
                "alg_bytes_per_launch": nbytes, "avg_launch_us": round(us, 3)}

    # The attention kernel alone (it moves the routed K/V, almost all of a
    # step's bytes), and the whole step (one launch for small batches) against
    # the step's algorithmic bytes. The dominant kernel of the timed step is
    # the step's one kernel where it runs as one launch, else the attention.
    roofline_attend = roof("attend", attend_bytes, attend_us)
    roofline_attend["gathered_bytes_per_launch"] = gather_bytes
    roofline_attend["gathered_gbs"] = round(gather_bytes / (attend_us * 1e-6) / 1e9, 1)
    if tiles is not None:
        # the tile kernel is a (masked) MFMA contraction: the method's flops
        # (4 D per routed token) against the dense bf16 peak; the flops the
        # masked tiles execute, and the bytes of each tile's union, beside
        tf = tiles["alg_flops"] / (attend_us * 1e-6) / 1e12
        tf_exec = tiles["executed_flops"] / (attend_us * 1e-6) / 1e12
        staged_gbs = tiles["bytes"] / (attend_us * 1e-6) / 1e9
        cache = cache_read_rate(torch, dev)
        roofline_attend = {
            "kernel": "hga_attend_tiles", "bound": "mfma", "achieved": round(tf, 2),
            "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_MFMA_BF16_TFLOPS, 5), "traffic": None,
            "alg_flops_per_launch": tiles["alg_flops"],
            "executed_flops_per_launch": tiles["executed_flops"],
            "executed_tflops": round(tf_exec, 1),
            "executed_frac": round(tf_exec / PEAK_MFMA_BF16_TFLOPS, 4),
            "bytes_per_launch": tiles["bytes"],
            "gbs": round(staged_gbs, 1),
            "infinity_cache_read": cache,
            "gbs_over_cache_read": round(staged_gbs / cache["read_gbs"], 3),
            "tiles": tiles["tiles"], "union_groups_per_tile": tiles["union_groups_per_tile"],
            "avg_launch_us": round(attend_us, 3)}
    roofline_step = roof("decode_step", step_bytes, decode_us)
    roofline_step["launches"] = 1 if decode_one_launch else 2
    roofline = dict(roofline_step if decode_one_launch else roofline_attend)
    # step 1 in full: every key read once, every summary written once
    build_bytes = K0.numel() * esize + w.B * w.Hkv * (w.n_chunks + w.n_groups) * w.D * 4
    roofline_build = (roof("summaries", build_bytes, kern_us["build"]["avg"])
                      if "build" in kern_us else None)

    # Many queries per KV head (prefill): scoring is a dense MFMA contraction.
    mfma = None
    if w.Nq > 1 and w.dtype == "bf16" and (w.Hq // w.Hkv) * w.Nq >= 64:
        rows_all = w.B * w.Hq * w.Nq
        chunk_flops = 2 * w.D * w.n_chunks * rows_all                    # every chunk, every row
        cand_flops = 2 * w.D * int((c >= 0).sum()) * gpc                  # the method's candidates
        executed = 2 * (2 * w.D * (w.n_chunks + w.n_groups) * rows_all)   # dense, hi and lo passes
        route_us = kern_us["route"]["avg"]
        alg = chunk_flops + cand_flops
        mfma = {"kernels": "route call: split + route_prefill_fused (MFMA scoring, both selections)",
                "alg_flops": alg, "chunk_gemm_flops": chunk_flops, "executed_flops": executed,
                "route_us": round(route_us, 2), "peak_tflops": PEAK_MFMA_BF16_TFLOPS,
                "achieved_tflops": round(alg / (route_us * 1e-6) / 1e12, 2),
                "frac": round(alg / (route_us * 1e-6) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 5),
                "achieved_tflops_executed": round(executed / (route_us * 1e-6) / 1e12, 1),
                "frac_executed": round(executed / (route_us * 1e-6) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
                "counters": stored_counters_note("route_prefill", w.name),
                "note": "time of the whole route call (split, scoring, selections)"}

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "accumulate": "f32",
        "data": "synthetic (seeded Gaussian Q/K/V, RoPE, planted q-aligned chunks)",
        "config": {"workload": w.name, "batch": w.B, "seq_len": w.T, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.D, "chunk": w.chunk, "group": w.group,
                   "k_chunk": w.k_chunk, "k_group": w.k_group,
                   "routed_fraction": round(routed_tokens / (rows * w.T), 5),
                   "cold_cache_copies": S, "hip_graph": use_graph,
                   "step": ("route_fresh_ex + attend_staged (newest-keys summary refresh + "
                            "routing, then attention over the distinct routed groups staged once)"
                            if w.host_kv else
                            "decode_step_ex (newest-keys summary refresh + routing + attention)")},
        "hbm_gbs_step": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "alg_bytes_per_step": step_bytes,
        "roofline": roofline,
        "roofline_attend": roofline_attend,
        "roofline_step": roofline_step,
        "roofline_build": roofline_build,
        "kernels_us": {k: round(v["avg"], 3) for k, v in kern_us.items()},
        "latency_us": {"p50": round(pct(lat, 0.5), 2), "p95": round(pct(lat, 0.95), 2),
                       "p99": round(pct(lat, 0.99), 2)},
        "warm_cache": warm,
        "setup_s": {"generate": round(t_gen, 1)},
    }
    if quality is not None:
        out["quality_vs_dense"] = quality
    if host is not None:
        out["host_tier"] = host
    out["mfma"] = mfma
    del sets, graphs_keep
    return out


PHASES = ["start", "scoring item done", "wave 0: the row's older chunk words in LDS",
          "chunk level selected and every score word in", "group level selected, ids in LDS",
          "wave 0's routed K/V folded in", "every wave's routed K/V folded in",
          "split 0: the other splits' partials in", "split 0: hand-off words zeroed, splits merged",
          "end of the workgroup", "wave 0: chunk level selected", "wave 0: group level selected"]


def decode_phases(w, steps):
    """Clock stamps (100 MHz, chip-wide) at the end of each phase of the
    one-launch decode step, from the phase-stamp build of the library: per
    phase, the earliest, median and latest workgroup, in us after the step's
    first workgroup started; medians over `steps` cold-cache steps."""
    import ctypes

    import numpy as np
    import torch

    import hierarchical_sparse_attention_summaries_amd as hga
    from synth import generate

    L = hga.lib()
    if not hasattr(L, "hga_debug_phase_stamps"):
        sys.exit("bench.py --phases needs the phase-stamp build: run "
                 "`python hierarchical_sparse_attention_summaries_amd/build.py --phase-stamps` "
                 "and set HGA_LIB=hierarchical_sparse_attention_summaries_amd/libhga_phases.so")
    L.hga_debug_phase_stamps.argtypes = [ctypes.c_void_p]
    L.hga_debug_phase_stamps.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    inp = generate(w, seed=0)
    Q = torch.from_numpy(inp.Q).to(dev, tdt)
    K0 = torch.from_numpy(inp.K).to(dev, tdt)
    V0 = torch.from_numpy(inp.V).to(dev, tdt)
    cm0, gm0 = hga.build_summaries(K0, w.chunk, w.group)
    shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
    if not hga.decode_step_one_launch(shape, w.dtype, w.chunk, w.group, w.k_chunk, w.k_group):
        sys.exit(f"{w.name}: the decode step is not one launch here")
    S = 15       # cold caches: rotate over copies, as the timed benchmark does
    sets = [(K0, V0, cm0, gm0)] + [(K0.clone(), V0.clone(), cm0.clone(), gm0.clone())
                                   for _ in range(S - 1)]
    ws = torch.zeros(hga.decode_step_workspace_bytes(shape, w.chunk, w.group, w.k_chunk,
                                                     w.k_group), dtype=torch.uint8, device=dev)

    def step(s):
        K, V, cm, gm = sets[s]
        hga.decode_step_ex(Q, K, V, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group,
                           workspace=ws)

    for k in range(30):
        step(k % S)
    torch.cuda.synchronize()
    stamps = torch.zeros(4096 * 16, dtype=torch.int64, device=dev)
    if L.hga_debug_phase_stamps(ctypes.c_void_p(stamps.data_ptr())) != 0:
        sys.exit("could not set the phase-stamp buffer")
    per = {k: [] for k in range(len(PHASES))}
    grid = 0
    for rep in range(steps):
        stamps.zero_()
        step(rep % S)
        torch.cuda.synchronize()
        a = stamps.view(-1, 16).cpu().numpy()
        a = a[a[:, 0] > 0]
        grid = len(a)
        rel = (a - a[:, 0].min()) * 0.01      # 100 MHz ticks -> us
        for k in range(len(PHASES)):
            ok = a[:, k] > 0
            if ok.any():
                v = rel[ok, k]
                per[k].append((float(v.min()), float(np.median(v)), float(v.max())))
    L.hga_debug_phase_stamps(None)
    out = {}
    for k, name in enumerate(PHASES):
        if per[k]:
            out[f"{k} {name}"] = {q: round(statistics.median(x[j] for x in per[k]), 2)
                                  for j, q in enumerate(("min", "median", "max"))}
    return {"workload": w.name, "steps": steps, "workgroups": grid,
            "unit": "us after the step's first workgroup started", "phases": out}


def quality_proxy(hga, torch, w, Q, K, V, gidx):
    """Synthetic stand-in for a quality comparison with dense attention: the
    same kernel run over every group (dense causal attention) next to the routed
    run. Per query head: the share of the dense softmax mass that lies on the
    routed tokens (exp(lse_routed - lse_dense)), the relative L2 error of O, and
    the lse gap in nats."""
    all_g = torch.arange(w.n_groups, dtype=torch.int32, device=Q.device)
    all_g = all_g.expand(w.B, w.Hq, w.Nq, w.n_groups).contiguous()
    Od, lsed = hga.attend(Q, K, V, all_g, w.group)
    Or, lser = hga.attend(Q, K, V, gidx, w.group)
    torch.cuda.synchronize()
    mass = torch.exp(lser - lsed).flatten()
    err = ((Or.float() - Od.float()).norm(dim=-1) / Od.float().norm(dim=-1)).flatten()
    gap = (lsed - lser).flatten()
    return {"mass_on_routed_mean": round(float(mass.mean()), 5),
            "mass_on_routed_min": round(float(mass.min()), 5),
            "rel_err_O_mean": round(float(err.mean()), 5),
            "rel_err_O_max": round(float(err.max()), 5),
            "lse_gap_nats_mean": round(float(gap.mean()), 5),
            "routed_fraction": round(w.k_group * w.group / w.T, 5)}


# The oracle's workload for the forked CPU workers: set by the parent before
# the pool starts, inherited by every worker.
_CPU_JOB = None


def _cpu_worker(seconds):
    """Complete decode steps of the oracle, as it stands, in one thread, for
    about `seconds`: the newest chunk's summaries recomputed, then routing and
    attention for every query head. Returns (steps, elapsed seconds, step times)."""
    from threadpoolctl import threadpool_limits

    import oracle

    w, inp, cm0, gm0 = _CPU_JOB
    cm, gm = cm0.copy(), gm0.copy()
    c_first = (w.T - w.Nq) // w.chunk
    lo = c_first * w.chunk

    def one():
        cm_l, gm_l = oracle.build_summaries(inp.K[:, :, lo:], w.chunk, w.group)
        cm[:, :, c_first:] = cm_l
        gm[:, :, lo // w.group:] = gm_l
        _, gidx, _ = oracle.route(inp.Q, cm, gm, w.T, w.chunk, w.group, w.k_chunk, w.k_group)
        oracle.attend(inp.Q, inp.K, inp.V, gidx, w.group)

    with threadpool_limits(limits=1):
        one()  # warm-up
        times = []
        t_start = time.perf_counter()
        t_end = t_start + seconds
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            one()
            times.append(time.perf_counter() - t0)
        elapsed = time.perf_counter() - t_start
    return len(times), elapsed, times


def _cpu_run(w, seconds, workers):
    """Tokens/s of the oracle on `workers` single-threaded processes, each
    running whole decode steps of w concurrently (throughput = the sum of
    their rates)."""
    import multiprocessing

    import oracle
    from synth import generate

    global _CPU_JOB
    inp = generate(w, seed=0)
    cm, gm = oracle.build_summaries(inp.K, w.chunk, w.group)   # setup, untimed
    _CPU_JOB = (w, inp, cm, gm)
    try:
        if workers == 1:
            res = [_cpu_worker(seconds)]
        else:
            with multiprocessing.get_context("fork").Pool(workers) as pool:
                res = pool.map(_cpu_worker, [seconds] * workers)
    finally:
        _CPU_JOB = None
    rate = sum(n / el for n, el, _ in res)            # decode steps per second, all workers
    times = sorted(t for _, _, ts in res for t in ts)
    med = times[len(times) // 2]
    return {"value": round(w.B * w.Nq * rate, 2), "unit": "tokens/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{sum(n for n, _, _ in res)} full decode steps of {w.name} "
                      f"(all {w.B * w.Hq * w.Nq} query rows each; newest-chunk summary "
                      f"refresh + routing + attention) over {workers} single-threaded "
                      f"process(es) for ~{seconds:.0f} s, median step {med * 1e3:.1f} ms, "
                      f"fp64 NumPy"}


def cpu_baselines(w, seconds):
    """The CPU oracle on the host's cores (at most 16, the CPU share of one
    GPU), plus a one-thread pass at the batch-16 4K-context sweep point for
    scaling context."""
    from synth import SWEEP

    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(16, affinity))
    main = _cpu_run(w, seconds, workers)
    one = _cpu_run(SWEEP[4096], max(3.0, seconds / 3), 1)
    main["cpu_model"] = _cpu_model()
    main["cpus_in_affinity"] = affinity
    main["single_thread_b16_t4096"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    return main


def run_conditions(torch):
    """Device, software and clocks of this run."""
    import subprocess

    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    clocks = None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=30)
        if r.returncode == 0:
            d = json.loads(r.stdout)
            card = next(iter(d.values()))
            clocks = {k: v for k, v in card.items() if "clock" in k.lower()}
    except Exception:
        pass
    return {"device": props.name, "gfx": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "hbm_gib": round(props.total_memory / 2 ** 30, 1), "rocm": rocm,
            "hip": torch.version.hip, "torch": torch.__version__, "clocks": clocks,
            "cpu_model": _cpu_model()}


def host_memory_slope(points):
    """HBM held by the host-tier step (K/V in host memory) at several context
    lengths: bytes per context token, and the slope between the shortest and
    the longest."""
    rows = []
    for r in points:
        c, h = r["config"], r["host_tier"]
        ctx = c["batch"] * c["seq_len"]
        rows.append({"seq_len": c["seq_len"], "batch": c["batch"],
                     "hbm_bytes_resident": h["hbm_bytes_resident"],
                     "hbm_bytes_per_context_token": round(h["hbm_bytes_resident"] / ctx, 1),
                     "kv_bytes_in_host_memory": h["kv_bytes_in_host_memory"],
                     "fetched_bytes_per_token": h["fetched_bytes_per_token"],
                     "value": r["value"], "unit": r["unit"]})
    rows.sort(key=lambda x: x["seq_len"])
    a, b = rows[0], rows[-1]
    slope = (b["hbm_bytes_resident"] - a["hbm_bytes_resident"]) / (
        b["batch"] * b["seq_len"] - a["batch"] * a["seq_len"])
    return {"points": rows, "hbm_bytes_per_added_context_token": round(slope, 1),
            "kv_bytes_per_context_token_in_host_memory":
                round(b["kv_bytes_in_host_memory"] / (b["batch"] * b["seq_len"]), 1)}


def stored_counters_note(kernel: str, workload: str):
    """The derived line of a committed counter summary (profiles/), if any."""
    path = os.path.join(ROOT, "profiles", f"hga_{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^counters_json: (\{.*\})\s*$", open(path).read(), flags=re.M)
    return json.loads(m.group(1)) if m else None


def _cpu_model():
    """The host CPU as /proc/cpuinfo gives it: the model name (a virtual
    machine may shorten it, e.g. to the vendor and product line), with the
    family, model and stepping numbers and the logical CPU count beside it."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v
    except OSError:
        return None
    name = fields.get("model name")
    if name is None:
        return None
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return f"{name} ({ids}; {os.cpu_count()} logical CPUs)" if ids else name


if __name__ == "__main__":
    main()

// Step 2 of HGA (abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709), one workgroup per query row: the two levels exactly as stated.
// The workgroup scores the query against the summaries of chunks 0..L (L = the
// query's own chunk), keeps chunk 0, chunk L and the k_chunk best of the chunks
// between, then gathers and scores only the groups of the kept chunks and keeps
// the k_group best of them. Everything between the two summary reads stays in
// LDS, so a row costs two memory round trips and no workgroup waits for or
// hands data to another. Optionally it first refreshes the summaries of the
// sequence's newest chunks from K.
#pragma once

#include <algorithm>

#include "hga_device.h"
#include "hga_internal.h"
#include "hga_select.h"
#include "hga_summary.h"

namespace hga {
namespace rowroute {

constexpr int kThreads = 512;  // 8 waves
constexpr int kWaves = kThreads / kWave;

// Summary rows are scored in passes: lane l of wave w takes dims
// [(l % LPR) * 8, +8) of rows base + j * stride + l / LPR, j < NB, with all of a
// pass's loads in flight together. 16 lanes per row (D = 128) or 8 (D = 64).
template <int D, int NB>
struct RowPass {
  static constexpr int LPR = D / 8;
  static constexpr int RPS = kWave / LPR;        // rows per wave-step
  static constexpr int kStride = kWaves * RPS;   // rows per workgroup-step
  static constexpr int kRows = NB * kStride;     // rows per pass
  float4 v0[NB], v1[NB];

  __device__ __forceinline__ static int base() { return (threadIdx.x / kWave) * RPS; }
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int j = 0; j < NB; ++j) v0[j] = v1[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // Issues the loads of this pass's rows i in [lo, hi); other slots unchanged.
  template <typename RowPtr>
  __device__ __forceinline__ void load(int base0, int lo, int hi, RowPtr row_ptr) {
    const int lane = lane_id();
    const int col = (lane % LPR) * 8;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = base0 + j * kStride + lane / LPR;
      if (i >= lo && i < hi) {
        const float* src = row_ptr(i) + col;
        v0[j] = *reinterpret_cast<const float4*>(src);
        v1[j] = *reinterpret_cast<const float4*>(src + 4);
      }
    }
  }
  // Scores of this pass's rows below n: row i -> out[i] (LDS).
  __device__ __forceinline__ void dot(const float (&q)[8], int base0, int n, float* out) const {
    const int lane = lane_id();
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = base0 + j * kStride + lane / LPR;
      float d = q[0] * v0[j].x;
      d = fmaf(q[1], v0[j].y, d);
      d = fmaf(q[2], v0[j].z, d);
      d = fmaf(q[3], v0[j].w, d);
      d = fmaf(q[4], v1[j].x, d);
      d = fmaf(q[5], v1[j].y, d);
      d = fmaf(q[6], v1[j].z, d);
      d = fmaf(q[7], v1[j].w, d);
      d = group_sum<LPR>(d);
      if (i < n && (lane % LPR) == 0) out[i] = d;
    }
  }
};

// Scores summary rows from..n-1 for query q: row i -> out[i] (LDS). Rows below
// n_mem come from global memory (mem_row), the rest from LDS (lds_row): two
// pointer kinds kept apart so that every load is a plain global or LDS load.
template <int D, int NB, typename MemRow, typename LdsRow>
__device__ __forceinline__ void score_rows(const float (&q)[8], int from, int n, int n_mem,
                                           MemRow mem_row, LdsRow lds_row, float* out) {
  using P = RowPass<D, NB>;
  for (int base0 = P::base() + from; base0 < n; base0 += P::kRows) {
    P r;
    r.clear();
    r.load(base0, 0, min(n, n_mem), mem_row);
    r.load(base0, n_mem, n, lds_row);
    r.dot(q, base0, n, out);
  }
}

// Rows per pass of the two levels. A route grid of at most one workgroup per
// CU ("big" form) spends registers on latency: level 1's first pass of loads
// stays in flight across the summary refresh, and level 2 (272 candidate
// groups at a 64K context) takes one pass. Larger grids keep to 128 VGPRs so
// that two workgroups share a CU.
constexpr int kChunkPass = 8;
constexpr int kChunkPassLeanFresh = 4;  // leaves registers for the refresh's loads
constexpr int kGroupPassBig = 16;
constexpr int kGroupPassLean = 9;

// Top-k of n keys held in LDS (`score(i)` gives item i's float score), by one
// wave; writes the chosen item ids ascending to out[0..k) and returns how many.
// Every lane reads an item whatever n (its index clamped to n - 1; item 0 must
// be readable), so that the reads carry no branch and all issue together;
// items past n get key 0.
template <int E, typename ScoreOf>
__device__ __forceinline__ int wave_select(int n, int k, ScoreOf score, int* out) {
  const int lane = lane_id();
  const int last = n > 0 ? n - 1 : 0;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * kWave + lane;
    const float s = score(min(i, last));
    key[e] = i < n ? order_key(s) : 0u;
  }
  SelMask<E> chosen = 0;
  if (n <= k) {
#pragma unroll
    for (int e = 0; e < E; ++e) chosen |= static_cast<SelMask<E>>(key[e] != 0u) << e;
  } else {
    chosen = wave_top_k<E>(key, k);
  }
  int before = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool c = (chosen >> e) & 1u;
    const uint64_t m = ballot(c);
    if (c) out[before + bits_below(m)] = e * kWave + lane;
    before += __popcll(m);
  }
  return before;
}

// wave_select writing the chosen items' ids rather than their positions:
// item(i, id) returns item i's score and sets its id; the ids of the chosen
// items go, in ascending item order, to out[0..got) (LDS) and, when gout is
// not null, to gout[0..got) too. Returns got.
template <int E, typename Item>
__device__ __forceinline__ int wave_select_ids(int n, int k, Item item, int* out, int32_t* gout) {
  const int lane = lane_id();
  const int last = n > 0 ? n - 1 : 0;  // as wave_select: every lane reads an item
  uint32_t key[E];
  int id[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * kWave + lane;
    const float s = item(min(i, last), id[e]);
    key[e] = i < n ? order_key(s) : 0u;
  }
  SelMask<E> chosen = 0;
  if (n <= k) {
#pragma unroll
    for (int e = 0; e < E; ++e) chosen |= static_cast<SelMask<E>>(key[e] != 0u) << e;
  } else {
    chosen = wave_top_k<E>(key, k);
  }
  int before = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool c = (chosen >> e) & 1u;
    const uint64_t m = ballot(c);
    if (c) {
      const int at = before + bits_below(m);
      out[at] = id[e];
      if (gout) gout[at] = id[e];
    }
    before += __popcll(m);
  }
  return before;
}

// The two selections above with one key slot fewer per lane when the n items
// fit in it (E is sized for the larger of a route's two levels): one wave
// issues at most one instruction per four cycles, so every radix step costs
// what it issues, and a slot fewer saves that slot's compares and counts.
template <int E, typename ScoreOf>
__device__ __forceinline__ int wave_select_fit(int n, int k, ScoreOf score, int* out) {
  if constexpr (E > 1) {
    if (n <= (E - 1) * kWave) return wave_select<E - 1>(n, k, score, out);
  }
  return wave_select<E>(n, k, score, out);
}
template <int E, typename Item>
__device__ __forceinline__ int wave_select_ids_fit(int n, int k, Item item, int* out,
                                                   int32_t* gout) {
  if constexpr (E > 1) {
    if (n <= (E - 1) * kWave) return wave_select_ids<E - 1>(n, k, item, out, gout);
  }
  return wave_select_ids<E>(n, k, item, out, gout);
}

constexpr int kFreshChunks = 2;   // chunks a refresh of <= C newest keys can touch
constexpr int kFreshMaxGpc = 16;  // groups per chunk the refresh keeps in LDS

// Dynamic LDS bytes of route_row_body: chunk scores, candidate scores and
// group ids, kept chunks, and the chosen ids of either level.
inline size_t route_row_lds_bytes(int64_t n_c, int64_t cap, int64_t gpc, int k_c, int k_g) {
  const int64_t picks = std::max<int64_t>(k_c, std::min<int64_t>(k_g, cap * gpc));
  return static_cast<size_t>(n_c + 2 * cap * gpc + cap + picks) * 4;
}
inline size_t route_row_lds_bytes(const RouteArgs& a) {
  return route_row_lds_bytes(a.n_c, kept_capacity(a), a.gpc, a.k_c, a.k_g);
}
// Static LDS of route_row_body (bound), with and without the refresh.
inline size_t route_row_static_lds(int64_t D, bool fresh) {
  const int rows = fresh ? kFreshChunks + kFreshChunks * kFreshMaxGpc + kWaves : 3;
  return static_cast<size_t>(rows) * D * 4 + 64;
}
// Every workgroup of these launches stays within the LDS a workgroup may use
// without opting in to more.
constexpr size_t kRowRouteMaxLds = 65536;

template <typename TQ, int D, int E, bool FRESH, bool BIG>
__device__ __forceinline__ void route_row_body(const RouteArgs& a, int bid, float* s_dyn) {
  // LDS: chunk scores [n_c] | candidate scores [cap * gpc] | candidate group ids
  // [cap * gpc] | kept chunks [cap] | chosen [max]
  const int cap = kept_capacity(a);
  float* s_cs = s_dyn;
  float* s_gs = s_cs + a.n_c;
  int* s_gid = reinterpret_cast<int*>(s_gs + cap * a.gpc);
  int* s_kept = s_gid + cap * a.gpc;
  int* s_pick = s_kept + cap;
  __shared__ int s_n_kept, s_n_old;

  // Workgroups are dealt to the 8 XCDs round-robin by index; give every query
  // row of one (sequence, KV head) the same residue mod 8, so that the rows
  // sharing chunk summaries share an L2. Indices past the last unit idle.
  const int rpu = (a.Hq / a.Hkv) * a.Nq;  // rows per (sequence, KV head)
  const int xcd = bid % 8;
  const int k = bid / 8;
  const int unit = xcd + 8 * (k / rpu);
  if (unit >= a.B * a.Hkv) return;
  const int row = unit * rpu + k % rpu;  // rows of a unit are consecutive (head-major)
  const int i = row % a.Nq;
  const int bh = row / a.Nq;
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int kv = h / (a.Hq / a.Hkv);
  const int p = route_seq_len(a, b) - a.Nq + i;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  if (p < 0) {  // a query before the sequence's first key: nothing to route
    if (a.chunk_idx)
      for (int t = threadIdx.x; t < a.k_c + 2; t += kThreads)
        a.chunk_idx[static_cast<size_t>(row) * (a.k_c + 2) + t] = -1;
    for (int t = threadIdx.x; t < a.k_g; t += kThreads)
      a.group_idx[static_cast<size_t>(row) * a.k_g + t] = -1;
    return;
  }
  const int L = p / a.C;

  // this lane's 8 query dims, scaled
  float q[8];
  {
    const int col = (lane % (D / 8)) * 8;
    const size_t off = static_cast<size_t>(row) * D + col;
    if constexpr (sizeof(TQ) == 4) {
      float x0[4], x1[4];
      widen(ld16(static_cast<const float*>(a.Q) + off), x0);
      widen(ld16(static_cast<const float*>(a.Q) + off + 4), x1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q[e] = x0[e] * a.scale;
        q[4 + e] = x1[e] * a.scale;
      }
    } else {
      widen(ld16(static_cast<const uint16_t*>(a.Q) + off), q);
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] *= a.scale;
    }
  }
  const size_t bkv = static_cast<size_t>(b * a.Hkv + kv);
  const float* cm = a.chunk_mean + bkv * a.n_c * D;
  const float* gm = a.group_mean + bkv * a.n_g * D;

  // Level 1's first pass of chunk-summary loads (in the big form it goes out
  // now, before the refresh below; it skips the chunks the refresh rewrites).
  constexpr int kL1 = (FRESH && !BIG) ? kChunkPassLeanFresh : kChunkPass;
  using P1 = RowPass<D, kL1>;
  P1 pass1;
  pass1.clear();
  const int base1 = P1::base();
  const int c_fresh = FRESH ? max(0, route_seq_len(a, b) - a.Nq) / a.C : L + 1;
  auto mem_chunk = [&](int c) { return cm + static_cast<size_t>(c) * D; };
  if constexpr (BIG) pass1.load(base1, 0, min(L + 1, c_fresh), mem_chunk);

  // Refresh: the chunks holding the sequence's newest Nq keys are recomputed
  // from K (same bits as the summaries kernel), written out, and scored from
  // LDS. Every row of this (sequence, KV head) writes the same values.
  int cf = 1, cl = 0;  // refreshed chunk range (empty unless FRESH)
  __shared__ float s_fc[FRESH ? kFreshChunks : 1][D];
  __shared__ float s_fg[FRESH ? kFreshChunks * kFreshMaxGpc : 1][D];
  __shared__ float s_part[FRESH ? kWaves : 1][D];
  using KR = KeyRowLoads<TQ, D>;
  constexpr int EPL = KR::EPL;
  const int Tb = route_seq_len(a, b);
  float* cm_w = const_cast<float*>(cm);
  float* gm_w = const_cast<float*>(gm);
  // Early refresh: when all the new keys lie in one chunk (always so in
  // decode), that chunk is every row's own chunk L, which is kept whatever its
  // score, so level 1 needs nothing from the refresh. Wave w then issues the
  // key loads of that chunk's group w first (the lean form, which keeps to 128 VGPRs,
  // scores level 1 in smaller passes to leave room for them), they stay in
  // flight while level 1 scores the older chunks, and the waves fold them
  // while wave 0 ranks the chunks (wave 0 folds its own after). Same rows,
  // lanes and order as chunk_summary, so the same bits.
  bool early = false;
  int g_first = 0, n_fg = 0, fg_rows = 0;
  KR fresh_rows;
  auto issue_fresh = [&]() {
    fresh_rows.clear();
    if (wave < n_fg) {
      const int64_t off =
          group_rows(a.kv, b, a.Hkv, kv, a.T, D, Tb, a.G, g_first + wave, &fg_rows);
      if (off >= 0) fresh_rows.issue(static_cast<const TQ*>(a.K) + off, 0, fg_rows);
    }
  };
  if constexpr (FRESH) {
    cf = max(0, Tb - a.Nq) / a.C;
    cl = (Tb - 1) / a.C;
    g_first = cf * a.gpc;
    n_fg = min(g_first + a.gpc, (Tb + a.G - 1) / a.G) - g_first;
    early = cf == cl && n_fg <= kWaves && a.G <= KR::kRows;
    if (early) issue_fresh();
  }
  // folds this wave's early-refresh group: mean to LDS, sum to s_part (the
  // means go to memory at the end: on gfx950 a wait for loads also waits for
  // every store issued before them, so stores here would hold up level 2)
  auto fold_fresh = [&]() {
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    fresh_rows.add_to(acc);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = across_rows_sum<KR::LPR>(acc[e]);
    const int col = (lane % KR::LPR) * EPL;
    if (lane / KR::LPR == 0) {
      if (wave < n_fg) {
        const int g = g_first + wave;
        const float inv = 1.f / static_cast<float>(fg_rows);
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_fg[g - cf * a.gpc][col + e] = acc[e] * inv;
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_part[wave][col + e] = 0.f + (wave < n_fg ? acc[e] : 0.f);
    }
  };
  if constexpr (FRESH) {
    for (int c = cf; c <= cl && !early; ++c) {
      chunk_summary<TQ, D, kWaves>(
          static_cast<const TQ*>(a.K), a.kv, b, a.Hkv, kv, a.T, Tb, a.C, a.G, c, s_part,
          [&](int g, int col, const float (&sum)[EPL], int count) {
            const float inv = 1.f / static_cast<float>(count);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              const float m = sum[e] * inv;
              gm_w[static_cast<size_t>(g) * D + col + e] = m;
              s_fg[g - cf * a.gpc][col + e] = m;
            }
          },
          [&](int d, float sum, int count) {
            const float m = sum / static_cast<float>(count);
            cm_w[static_cast<size_t>(c) * D + d] = m;
            s_fc[c - cf][d] = m;
          });
      __syncthreads();
    }
  }
  // chunks below c_fresh from memory, the refreshed ones (c_fresh..L) from LDS
  auto lds_chunk = [&](int c) { return &s_fc[FRESH ? c - cf : 0][0]; };

  // Level 1: chunks 0..L (0..L-1 after an early refresh: chunk L's score is
  // never used, and its summary is not ready yet).
  const int n_l1 = early ? L : L + 1;
  if constexpr (!BIG) pass1.load(base1, 0, min(n_l1, c_fresh), mem_chunk);
  pass1.load(base1, c_fresh, n_l1, lds_chunk);
  pass1.dot(q, base1, n_l1, s_cs);
  score_rows<D, kL1>(q, P1::kRows, n_l1, c_fresh, mem_chunk, lds_chunk, s_cs);
  __syncthreads();
  if (FRESH && early && wave != 0) fold_fresh();
  if (wave == 0) {
    int n_kept;
    if (L + 1 <= a.k_c + 2) {
      n_kept = L + 1;
      for (int t = lane; t < n_kept; t += kWave) s_kept[t] = t;
    } else {
      n_kept = a.k_c + 2;
      const int got = a.k_c > 0 ? wave_select_fit<E>(L - 1, a.k_c,
                                                     [&](int t) { return s_cs[1 + t]; }, s_pick)
                                : 0;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int t = lane; t < got; t += kWave) s_kept[1 + t] = 1 + s_pick[t];
      if (lane == 0) {
        s_kept[0] = 0;
        s_kept[n_kept - 1] = L;
      }
    }
    // kept chunks that were not refreshed (the kept list ascends)
    int n_old = 0;
    for (int t = lane; t < n_kept; t += kWave) n_old += s_kept[t] < c_fresh ? 1 : 0;
    n_old = static_cast<int>(wave_add(static_cast<uint32_t>(n_old)));
    if (lane == 0) {
      s_n_kept = n_kept;
      s_n_old = n_old;
    }
    if (FRESH && early) fold_fresh();
  }
  __syncthreads();
  if (FRESH && early && static_cast<int>(threadIdx.x) < D) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += s_part[w][threadIdx.x];
    s_fc[0][threadIdx.x] = sum / static_cast<float>(min(a.C, Tb - cf * a.C));
  }
  const int n_kept = s_n_kept;
  // candidate t (in kept-chunk order) is group s_gid[t]
  for (int t = threadIdx.x; t < n_kept * a.gpc; t += kThreads)
    s_gid[t] = s_kept[t / a.gpc] * a.gpc + t % a.gpc;
  if (a.chunk_idx) {
    for (int t = threadIdx.x; t < a.k_c + 2; t += kThreads)
      a.chunk_idx[static_cast<size_t>(row) * (a.k_c + 2) + t] = t < n_kept ? s_kept[t] : -1;
  }

  // Level 2: the groups of the kept chunks that start at or before p.
  const int n_cand = n_kept * a.gpc;
  auto valid = [&](int t) {
    const int g = s_gid[t];
    return g < a.n_g && static_cast<int64_t>(g) * a.G <= p;
  };
  __syncthreads();
  score_rows<D, BIG ? kGroupPassBig : kGroupPassLean>(
      q, 0, n_cand, s_n_old * a.gpc,
      [&](int t) {
        const int g = s_gid[t];
        return gm + static_cast<size_t>(g < a.n_g ? g : 0) * D;
      },
      [&](int t) { return &s_fg[FRESH ? s_gid[t] - cf * a.gpc : 0][0]; }, s_gs);
  __syncthreads();
  if (FRESH && early && wave != 0) {  // the refreshed means, while wave 0 selects
    const int t0 = static_cast<int>(threadIdx.x) - kWave;
    for (int t = t0; t < n_fg * D; t += kThreads - kWave)
      gm_w[static_cast<size_t>(g_first) * D + t] = s_fg[t / D][t % D];
    for (int t = t0; t < D; t += kThreads - kWave) cm_w[static_cast<size_t>(cf) * D + t] = s_fc[0][t];
  }
  if (wave == 0) {
    // Invalid candidates sit only in the last kept chunk (after p or past the
    // end), i.e. at the end of the list: select among the valid prefix.
    int n_valid = 0;
    for (int t = lane; t < n_cand; t += kWave) n_valid += valid(t) ? 1 : 0;
    n_valid = static_cast<int>(wave_add(static_cast<uint32_t>(n_valid)));
    const int got = wave_select<E>(n_valid, a.k_g, [&](int t) { return s_gs[t]; }, s_pick);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    int32_t* out = a.group_idx + static_cast<size_t>(row) * a.k_g;
    for (int t = lane; t < a.k_g; t += kWave) out[t] = t < got ? s_gid[s_pick[t]] : -1;
  }
}


}  // namespace rowroute
}  // namespace hga

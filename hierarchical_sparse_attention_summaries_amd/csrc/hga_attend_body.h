// Step 3 of HGA (abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709): exact token-level softmax attention over the routed tokens only.
//
// Each query row (b, h, i) owns k_group routed groups. A wave takes
// `groups_per_wave` of them; for each group it gathers the group's keys and
// values (a group is G consecutive rows, in a dense cache or within one page;
// 16-byte coalesced loads; the next group's loads in flight while the current
// one is folded in) into an online softmax (running max m, sum l and output o
// in fp32, exponentials in base 2 with log2(e) folded into the query). The
// four waves of a workgroup merge in LDS; the workgroups of a row (split-K over
// its groups) leave (m, l, o) partials and the last one to arrive merges them
// and writes O and lse. HBM-bound: every routed K/V byte is read once.
#pragma once

#include <math.h>

#include "hga_device.h"
#include "hga_internal.h"

namespace hga {

constexpr int kAttendThreads = 256;
constexpr int kAttendWaves = kAttendThreads / kWave;
constexpr int kAttendTile = 32;        // tokens per gather tile
constexpr int kAttendMaxSplits = 32;   // workgroups per row at most (the plan guarantees it)

struct NoRowHook {
  __device__ void operator()() const {}
};

// One attention workgroup: row `row_base + bid / n_splits`, split
// `bid % n_splits`. With LDS_IDS the row's group ids are already in LDS
// (s_ids, k_group entries), chosen by this workgroup itself; `poisoned` then
// marks a row whose routing could not be completed (its outputs become NaN).
// `row_done` is called by every thread of the workgroup that finishes the row,
// as soon as every split of the row has counted itself in (so every split is
// past everything it did before its partial sums).
// With POLL_MERGE (every workgroup of the row resident at once), the partials
// go to memory that is zero at rest as hand-off words instead: splits 1.. store
// theirs and are done, and split 0 polls them (bounded; NaN outputs if one
// does not arrive in time), merges, and zeroes them again; no counters.
// Returns true in the workgroup that wrote the row's outputs.
template <typename TKV, int D, int WAVES = kAttendWaves, bool LDS_IDS = false,
          typename RowHook = NoRowHook, bool POLL_MERGE = false>
__device__ __forceinline__ bool attend_body(const AttendArgs& a, int groups_per_wave, int n_splits,
                                            int row_base, int bid, const int* s_ids = nullptr,
                                            bool poisoned = false, RowHook row_done = RowHook{}) {
  constexpr int kBodyThreads = WAVES * kWave;
  constexpr int EPL = Elem<TKV>::kPer16;
  constexpr int LPR = D / EPL;        // lanes per token row
  constexpr int RPL = kWave / LPR;    // token rows per wave-wide load
  constexpr int NLD = kAttendTile / RPL;    // loads per tile (per K and per V)
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.6931471805599453f;

  __shared__ float s_m[WAVES], s_l[WAVES];
  __shared__ float s_o[WAVES][D];
  __shared__ bool s_last;
  __shared__ float s_part[kAttendMaxSplits * (D + 2)];

  const int row = row_base + bid / n_splits;
  const int split = bid % n_splits;
  const int i = row % a.Nq;
  const int bh = row / a.Nq;
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int kv = h / (a.Hq / a.Hkv);
  const int p = seq_len_of(a.kv, b, a.T) - a.Nq + i;
  const int t_lim = p + 1;  // tokens j <= p (p < the sequence's length <= T); none if p < 0
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int sub = lane / LPR;
  const int col = (lane % LPR) * EPL;

  const TKV* Kbase = static_cast<const TKV*>(a.K);
  const TKV* Vbase = static_cast<const TKV*>(a.V);

  float q[EPL];
  {
    widen(ld16(static_cast<const TKV*>(a.Q) + static_cast<size_t>(row) * D + col), q);
    const float s = a.scale * kLog2e;
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[e] *= s;
  }

  float m = -INFINITY, l = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;

  const int32_t* gl = a.group_idx + static_cast<size_t>(row) * a.k_g;
  bool timed_out = poisoned;
  const int e0 = (split * WAVES + wave) * groups_per_wave;
  const int e1 = min(e0 + groups_per_wave, a.k_g);
  const int n_g = (a.T + a.G - 1) / a.G;

  // The wave's list entries, 64 at a time: lane j holds entry gb + j, all
  // loaded at once (one memory round trip instead of one per group).
  int gb = e0 - kWave;
  int g_lane = -1;
  auto entry = [&](int e) -> int {  // e is the same in every lane
    if (e >= gb + kWave) {
      gb += kWave;
      const int j = gb + lane_id();
      if (j < e1) {
        if constexpr (LDS_IDS) {
          g_lane = s_ids[j];
        } else {
          g_lane = gl[j];
        }
      } else {
        g_lane = -1;
      }
    }
    return __builtin_amdgcn_readlane(g_lane, e - gb);
  };

  // Token range [t0, t1) of list entry e (empty for -1 padding, ids out of
  // range, groups that start after the query, and pages out of range), and the
  // element offset of its first row: the group's rows are consecutive.
  auto span = [&](int e, int& t0, int& t1, int64_t& off) {
    const int g = e < e1 ? entry(e) : -1;
    t0 = t1 = 0;
    off = 0;
    if (g < 0 || g >= n_g) return;
    const int s0 = g * a.G;
    const int s1 = min(s0 + a.G, t_lim);
    if (s1 <= s0) return;
    off = kv_offset(a.kv, b, a.Hkv, kv, a.T, D, s0);
    if (off < 0) return;
    t0 = s0;
    t1 = s1;
  };
  // Issue the loads of up to kAttendTile tokens from `base` (rows >= t1 read as
  // 0): buffers over rows [base, t1) of the group, so no load sits in a branch.
  auto load = [&](int base, int t1, int64_t off, int t0, uint4 (&kr)[NLD], uint4 (&vr)[NLD]) {
    const int bytes = max(0, t1 - base) * D * static_cast<int>(sizeof(TKV));
    const int64_t at = off + static_cast<int64_t>(base - t0) * D;  // row `base` of the group
    const __amdgpu_buffer_rsrc_t rk = buffer_of(Kbase + at, bytes);
    const __amdgpu_buffer_rsrc_t rv = buffer_of(Vbase + at, bytes);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int off_b = ((u * RPL + sub) * D + col) * static_cast<int>(sizeof(TKV));
      kr[u] = buffer_ld16(rk, off_b);
      vr[u] = buffer_ld16(rv, off_b);
    }
  };
  // Fold one loaded tile into (m, l, o). Token `base` must be valid.
  auto consume = [&](int base, int t1, const uint4 (&kr)[NLD], const uint4 (&vr)[NLD]) {
    float sc[NLD];
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      float x[EPL];
      widen(kr[u], x);
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) d = fmaf(q[k], x[k], d);
      d = group_sum<LPR>(d);
      sc[u] = (base + u * RPL + sub < t1) ? d : -INFINITY;
      mt = fmaxf(mt, sc[u]);
    }
    mt = across_rows_max<LPR>(mt);
    const float m_new = fmaxf(m, mt);  // finite: token `base` is valid
    const float corr = exp2f(m - m_new);
    l *= corr;
#pragma unroll
    for (int k = 0; k < EPL; ++k) o[k] *= corr;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const float pu = exp2f(sc[u] - m_new);
      l += pu;
      float x[EPL];
      widen(vr[u], x);
#pragma unroll
      for (int k = 0; k < EPL; ++k) o[k] = fmaf(pu, x[k], o[k]);
    }
    m = m_new;
  };

  // fp32 groups in 512-thread workgroups (256 VGPRs at most): one buffer, so
  // that the tile does not spill
  constexpr bool kDouble = !(sizeof(TKV) == 4 && kBodyThreads > kAttendThreads);
  if (kDouble && a.G <= kAttendTile) {
    // One tile per group. Two register buffers: the next group's keys and
    // values are in flight while the current one is folded in.
    uint4 kA[NLD], vA[NLD], kB[NLD], vB[NLD];
    int a0, a1, b0, b1;
    int64_t ao, bo;
    span(e0, a0, a1, ao);
    load(a0, a1, ao, a0, kA, vA);
    for (int e = e0; e < e1; e += 2) {
      span(e + 1, b0, b1, bo);
      load(b0, b1, bo, b0, kB, vB);
      if (a0 < a1) consume(a0, a1, kA, vA);
      span(e + 2, a0, a1, ao);
      load(a0, a1, ao, a0, kA, vA);
      if (b0 < b1) consume(b0, b1, kB, vB);
    }
  } else {
    // Groups longer than a tile (or one buffer only): walk the tiles one by one.
    uint4 kA[NLD], vA[NLD];
    for (int e = e0; e < e1; ++e) {
      int t0, t1;
      int64_t off;
      span(e, t0, t1, off);
      for (int base = t0; base < t1; base += kAttendTile) {
        load(base, t1, off, t0, kA, vA);
        consume(base, t1, kA, vA);
      }
    }
  }
#ifdef HGA_PHASE
  HGA_PHASE(5);  // wave 0's groups folded in
#endif
  // Lanes of one column slot hold disjoint token rows: fold them.
  l = across_rows_sum<LPR>(l);
#pragma unroll
  for (int k = 0; k < EPL; ++k) o[k] = across_rows_sum<LPR>(o[k]);
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = l;
  }
  if (threadIdx.x == 0) s_last = true;
  if (sub == 0) {
#pragma unroll
    for (int k = 0; k < EPL; ++k) s_o[wave][col + k] = o[k];
  }
  __syncthreads();
#ifdef HGA_PHASE
  HGA_PHASE(6);  // every wave's groups folded in
#endif

  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w]);
  float Lsum = 0.f, acc = 0.f;
  const int d = threadIdx.x;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float f = exp2f(s_m[w] - M);
      Lsum += s_l[w] * f;
      if (d < D) acc += s_o[w][d] * f;
    }
  }
  // A split that gave up waiting poisons its row (NaN survives the merge).
  if (timed_out) Lsum = __builtin_nanf("");

  auto finish = [&](float Mx, float Lx, float ox) {
    if (timed_out) {
      Lx = 1.f;
      ox = __builtin_nanf("");
    }
    if (d < D) {
      const float v = Lx > 0.f ? ox / Lx : 0.f;
      const size_t off = static_cast<size_t>(row) * D + d;
      if constexpr (sizeof(TKV) == 4) {
        static_cast<float*>(a.O)[off] = v;
      } else {
        static_cast<uint16_t*>(a.O)[off] = static_cast<uint16_t>(bf16_bits(v));
      }
    }
    if (a.lse && d == 0)
      a.lse[row] = timed_out ? __builtin_nanf("") : Lx > 0.f ? (Mx + log2f(Lx)) * kLn2 : -INFINITY;
  };

  if (n_splits == 1) {
    row_done();
    finish(M, Lsum, acc);
    return true;
  }
  if constexpr (POLL_MERGE) {
    int32_t* slots = reinterpret_cast<int32_t*>(a.partials) +
                     static_cast<size_t>(row) * n_splits * (D + 2);
    if (split != 0) {
      int32_t* mine = slots + split * (D + 2);
      if (d < D) store_shared_i32(mine + 2 + d, handoff_word(acc));
      if (d == 0) {
        store_shared_i32(mine, handoff_word(M));
        store_shared_i32(mine + 1, handoff_word(Lsum));
      }
      return false;
    }
    // split 0: its own partial goes to slot 0 in LDS, the others' as they land
    if (d < D) s_part[2 + d] = acc;
    if (d == 0) {
      s_part[0] = M;
      s_part[1] = Lsum;
    }
    const int total = (n_splits - 1) * (D + 2);
    bool arrived = true;
    for (int base = 0; base < total; base += 4 * kBodyThreads) {
      int32_t v[4];
      unsigned pending = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * kBodyThreads + threadIdx.x;
        v[u] = idx < total ? load_shared_i32(slots + D + 2 + idx) : 1;
        pending |= static_cast<unsigned>(v[u] == 0) << u;
      }
      for (int it = 0; pending != 0u && it < (1 << 20); ++it) {
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = base + u * kBodyThreads + threadIdx.x;
          if ((pending >> u) & 1u) v[u] = load_shared_i32(slots + D + 2 + idx);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) pending &= ~(static_cast<unsigned>(v[u] != 0) << u);
      }
      arrived = arrived && pending == 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * kBodyThreads + threadIdx.x;
        if (idx < total) s_part[D + 2 + idx] = handoff_float(v[u]);
      }
    }
    if (!arrived) {
      s_last = false;
      if (a.status) store_shared_i32(a.status, kStatusTimedOut);
    }
    __syncthreads();
#ifdef HGA_PHASE
    HGA_PHASE(7);  // the other splits' partials in
#endif
    if (!s_last) timed_out = true;
    // every other split has stored its partial, so is past the row's scores
    row_done();
    for (int idx = threadIdx.x; idx < total; idx += kBodyThreads)
      store_shared_i32(slots + D + 2 + idx, 0);
  } else {
    float* part = a.partials + (static_cast<size_t>(row) * n_splits + split) * (D + 2);
    if (d < D) store_shared(part + 2 + d, acc);
    if (d == 0) {
      store_shared(part, M);
      store_shared(part + 1, Lsum);
    }
    if (!arrive_last(a.counters + (row - row_base), static_cast<unsigned>(n_splits), &s_last))
      return false;
    row_done();

    // Pull every split's (m, l, o) into LDS with all loads in flight at once.
    const float* rp = a.partials + static_cast<size_t>(row) * n_splits * (D + 2);
    const int total = n_splits * (D + 2);
    for (int base = 0; base < total; base += 4 * kBodyThreads) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * kBodyThreads + threadIdx.x;
        v[u] = idx < total ? load_shared(rp + idx) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * kBodyThreads + threadIdx.x;
        if (idx < total) s_part[idx] = v[u];
      }
    }
    __syncthreads();
  }
  // The splits' (m, l, o) in blocks of kMB splits, each block's LDS reads
  // issued together: one LDS round trip per block rather than per split. The
  // sums run in split order, as one split at a time would.
  constexpr int kMB = 8;
  float Mx = -INFINITY;
  for (int s0 = 0; s0 < n_splits; s0 += kMB) {
    float mv[kMB];
#pragma unroll
    for (int j = 0; j < kMB; ++j) mv[j] = s_part[min(s0 + j, kAttendMaxSplits - 1) * (D + 2)];
#pragma unroll
    for (int j = 0; j < kMB; ++j)
      if (s0 + j < n_splits) Mx = fmaxf(Mx, mv[j]);
  }
  float Lx = 0.f, ox = 0.f;
  if (Mx != -INFINITY) {
    for (int s0 = 0; s0 < n_splits; s0 += kMB) {
      float mv[kMB], lv[kMB], ov[kMB];
#pragma unroll
      for (int j = 0; j < kMB; ++j) {
        const float* ps = &s_part[min(s0 + j, kAttendMaxSplits - 1) * (D + 2)];
        mv[j] = ps[0];
        lv[j] = ps[1];
        ov[j] = d < D ? ps[2 + d] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kMB; ++j) {
        if (s0 + j < n_splits) {
          const float f = exp2f(mv[j] - Mx);
          Lx += lv[j] * f;
          ox += ov[j] * f;
        }
      }
    }
  }
#ifdef HGA_PHASE
  HGA_PHASE(8);  // merged
#endif
  finish(Mx, Lx, ox);
  return true;
}


}  // namespace hga

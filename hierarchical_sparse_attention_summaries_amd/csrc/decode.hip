// One decode step of HGA (abstract of "Hierarchical Global Attention (HGA)",
// arXiv 2606.30709) as a single launch: refresh the newest chunk summaries,
// score, select, attend.
//
// The grid is at most one workgroup per CU, all resident at once, and every
// workgroup plays two parts in turn. A "unit" is one sequence's KV head (U =
// B * Hkv of them), shared by its r * Nq query rows.
//
// Scoring item (workgroups [0, U * items)): the summaries of a unit are scored
// against all of the unit's query rows at both levels at once: every chunk and
// every group, so that no level waits for the other. Item 0 of a unit
// recomputes the chunks holding the sequence's newest keys from K (same bits
// as the summaries kernel), writes them out and scores them; the others split
// the older summaries evenly. Scores go to the workspace's zero-at-rest region
// with agent-coherent stores, as words that are never zero (handoff_word), so a
// score that has arrived is its own ready signal: no flag, no wait for the
// stores to be acknowledged, no second read. Scoring never waits.
//
// Attention item (workgroups [0, rows * n_splits)): the workgroup polls its
// row's score words (bounded) until none is zero and decodes them into LDS,
// and wave 0 makes the row's two-level selection (every split of the row
// chooses the same ids from the same scores); then 8 waves gather the split's
// share of the routed keys and values. Split 0 writes the row's ids out. The
// workgroup that finishes a row (every split has counted itself in, so every
// split has read the row's scores) zeroes the row's score words for the next
// call. The splits' partial sums go the same way: splits 1.. leave them as
// hand-off words in the zero-at-rest region and split 0 polls, merges and
// zeroes them, so the step uses no counter at all.
//
// Against one workgroup per query row running both levels back to back, this
// reads every group summary (not only the candidates'), spread over every CU,
// and saves the group level's dependent summary reads and the hand-over of
// the ids between routing and attention.
#include <hip/hip_runtime.h>

// Phase stamps (a separate build with HGA_PHASE_STAMPS defined; off in the
// library): thread 0 of every workgroup writes the chip-wide 100 MHz clock at
// the end of each phase of the step to a buffer the host sets, slot
// 16 * workgroup + phase.
#ifdef HGA_PHASE_STAMPS
__device__ unsigned long long* g_hga_phase_stamps;
#define HGA_PHASE(k)                                                                    \
  do {                                                                                  \
    if (threadIdx.x == 0 && g_hga_phase_stamps)                                         \
      g_hga_phase_stamps[blockIdx.x * 16 + (k)] = __builtin_amdgcn_s_memrealtime();     \
  } while (0)
#else
#define HGA_PHASE(k) \
  do {               \
  } while (0)
#endif

#include "hga_attend_body.h"
#include "hga_route_row_body.h"

namespace hga {
namespace {

using rowroute::kThreads;
using rowroute::kWaves;

struct StepArgs {
  int32_t* scores;    // [rows, n_c + n_g] score words (chunks, then groups); zero at rest
  int items;          // scoring items per unit (>= 2)
  int n_splits;       // attention workgroups per row
  int groups_per_wave;
};

// Score words a scoring pass writes for each query row of a unit whose
// sequence holds Tb > 0 keys: chunks [0, n_chunks), groups [0, n_groups). The
// newest chunk cl is always kept (a row's own chunk, L <= cl) and the chunk
// level ranks chunks 1..L-1 only, so its score is never needed or written.
__device__ __forceinline__ void written_range(const RouteArgs& a, int Tb, int& n_chunks,
                                              int& n_groups) {
  const int cl = (Tb - 1) / a.C;
  n_chunks = cl;
  n_groups = min((cl + 1) * a.gpc, (Tb + a.G - 1) / a.G);
}

// The unit's query rows, scaled, for the scoring: with nq <= kPreQ rows they
// are staged once per workgroup in LDS (thread t holds 8 dims of row
// t / (D / 8) in flight from q_issue until q_stage writes them), so that every
// lane reads them instead of loading and converting its own copy.
constexpr int kPreQ = 16;

template <typename TQ, int D>
__device__ __forceinline__ void q_issue(const RouteArgs& a, int row0, int nq, uint4& r0,
                                        uint4& r1) {
  constexpr int LPQ = D / 8;
  const int qj = threadIdx.x / LPQ, qcol = (threadIdx.x % LPQ) * 8;
  r0 = r1 = make_uint4(0, 0, 0, 0);
  if (qj < nq && qj < kPreQ) {
    const size_t off = static_cast<size_t>(row0 + qj) * D + qcol;
    if constexpr (sizeof(TQ) == 4) {
      r0 = ld16(static_cast<const float*>(a.Q) + off);
      r1 = ld16(static_cast<const float*>(a.Q) + off + 4);
    } else {
      r0 = ld16(static_cast<const uint16_t*>(a.Q) + off);
    }
  }
}

// q = widen(Q) * scale, the values the row route uses.
template <typename TQ>
__device__ __forceinline__ void q_scaled(const uint4& r0, const uint4& r1, float scale,
                                         float (&q)[8]) {
  if constexpr (sizeof(TQ) == 4) {
    float x0[4], x1[4];
    widen(r0, x0);
    widen(r1, x1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[e] = x0[e] * scale;
      q[4 + e] = x1[e] * scale;
    }
  } else {
    widen(r0, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] *= scale;
  }
}

template <typename TQ, int D>
__device__ __forceinline__ void q_stage(const RouteArgs& a, int nq, const uint4& r0,
                                        const uint4& r1, float (*s_q)[D]) {
  constexpr int LPQ = D / 8;
  const int qj = threadIdx.x / LPQ, qcol = (threadIdx.x % LPQ) * 8;
  if (qj < kPreQ) {  // rows nq.. are zero, so that readers need no bounds test
    float q[8];
    q_scaled<TQ>(r0, r1, a.scale, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) s_q[qj][qcol + e] = qj < nq ? q[e] : 0.f;
  }
}

// Scores summary rows i in [0, n) (row_ptr(i): D floats, all of one pointer
// kind) against query rows row0 .. row0 + nq - 1: the score of query row j and
// summary row i goes to scores[(row0 + j) * NS + col_of(i)] as a score word. Lane l of wave w
// holds dims [(l % LPR) * 8, +8) of summary rows w * RPS + l / LPR + k * kStride;
// the dot product is the row route's, in the same order, so both give the same
// bits. Waves without summary rows in a pass skip its arithmetic.
// Query rows: with s_q given (nq <= kPreQ), from LDS; `stage` then means that
// this call writes them there from q_issue's registers (r0, r1) once the first
// pass's summary loads are in flight (a workgroup barrier: every thread of the
// workgroup calls). Without s_q, every lane loads its rows from Q.
template <typename TQ, int D, typename RowPtr, typename ColOf>
__device__ __forceinline__ void score_block(const RouteArgs& a, int row0, int nq, int n,
                                            RowPtr row_ptr, ColOf col_of, int32_t* scores,
                                            int NS, float (*s_q)[D] = nullptr,
                                            bool stage = false,
                                            const uint4& r0 = make_uint4(0, 0, 0, 0),
                                            const uint4& r1 = make_uint4(0, 0, 0, 0)) {
  constexpr int LPR = D / 8;
  constexpr int RPS = kWave / LPR;
  constexpr int kStride = kWaves * RPS;
  constexpr int NB = 2;  // summary rows per lane per pass
  constexpr int QB = 8;  // query rows per pass
  const int lane = lane_id();
  const int col = (lane % LPR) * 8;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int first = wave * RPS + lane / LPR;
  for (int base = 0; base < n; base += NB * kStride) {
    const bool live = base + wave * RPS < n;  // the wave has rows in this pass
    float4 v0[NB], v1[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = base + first + j * kStride;
      if (live && i < n) {
        const float* src = row_ptr(i) + col;
        v0[j] = *reinterpret_cast<const float4*>(src);
        v1[j] = *reinterpret_cast<const float4*>(src + 4);
      } else {
        v0[j] = v1[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    if (stage && base == 0) {
      q_stage<TQ, D>(a, nq, r0, r1, s_q);
      __syncthreads();
    }
    if (!live) continue;
    for (int qb = 0; qb < nq; qb += QB) {
      float q[QB][8];
      if (s_q != nullptr) {  // all kPreQ rows are written (zero past nq)
#pragma unroll
        for (int r = 0; r < QB; ++r) {
          const float4 x0 = *reinterpret_cast<const float4*>(&s_q[qb + r][col]);
          const float4 x1 = *reinterpret_cast<const float4*>(&s_q[qb + r][col + 4]);
          q[r][0] = x0.x; q[r][1] = x0.y; q[r][2] = x0.z; q[r][3] = x0.w;
          q[r][4] = x1.x; q[r][5] = x1.y; q[r][6] = x1.z; q[r][7] = x1.w;
        }
      } else {
        // all of the pass's query loads in flight at once
        uint4 raw0[QB], raw1[QB];
#pragma unroll
        for (int r = 0; r < QB; ++r) {
          raw0[r] = raw1[r] = make_uint4(0, 0, 0, 0);
          if (qb + r < nq) {
            const size_t off = static_cast<size_t>(row0 + qb + r) * D + col;
            if constexpr (sizeof(TQ) == 4) {
              raw0[r] = ld16(static_cast<const float*>(a.Q) + off);
              raw1[r] = ld16(static_cast<const float*>(a.Q) + off + 4);
            } else {
              raw0[r] = ld16(static_cast<const uint16_t*>(a.Q) + off);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < QB; ++r) {
          q_scaled<TQ>(raw0[r], raw1[r], a.scale, q[r]);
          if (qb + r >= nq) {
#pragma unroll
            for (int e = 0; e < 8; ++e) q[r][e] = 0.f;
          }
        }
      }
      // partial dot products over this lane's 8 dims, value k = j * QB + r
      float part[NB * QB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int r = 0; r < QB; ++r) {
          float d = q[r][0] * v0[j].x;
          d = fmaf(q[r][1], v0[j].y, d);
          d = fmaf(q[r][2], v0[j].z, d);
          d = fmaf(q[r][3], v0[j].w, d);
          d = fmaf(q[r][4], v1[j].x, d);
          d = fmaf(q[r][5], v1[j].y, d);
          d = fmaf(q[r][6], v1[j].z, d);
          d = fmaf(q[r][7], v1[j].w, d);
          part[j * QB + r] = d;
        }
      }
      // Sum over the row's LPR lanes, scattered: lane t of the row ends with
      // value t (D = 128: all 16 values) or values t and QB + t (D = 64), each
      // with group_sum's bits; then every lane stores its own.
      static_assert(LPR * (LPR == 16 ? 1 : 2) == NB * QB, "values per row group");
      const int t = lane % LPR;
#pragma unroll
      for (int h = 0; h < NB * QB / LPR; ++h) {
        float c[LPR];
#pragma unroll
        for (int k = 0; k < LPR; ++k) c[k] = part[h * LPR + k];
        const float d = group_sum_scatter<LPR>(c);
        const int k = h * LPR + t;
        const int j = k / QB, r = k % QB;
        const int i = base + first + j * kStride;
        if (i < n && qb + r < nq)
          store_shared_i32(scores + static_cast<size_t>(row0 + qb + r) * NS + col_of(i),
                           handoff_word(d));
      }
    }
  }
}

// Refreshed summaries of a unit in LDS: chunk c at row c - cf, group g at row
// kFreshChunks + g - cf * gpc.
template <int D>
using FreshRows = float[rowroute::kFreshChunks * (1 + rowroute::kFreshMaxGpc)][D];

// Scoring item m of unit u (see the top of the file). Item 0 leaves the
// refreshed summaries in s_fr for write_refreshed.
template <typename TQ, int D>
__device__ __forceinline__ void score_item(const RouteArgs& a, const StepArgs& s, int u, int m,
                                           FreshRows<D>& s_fr) {
  __shared__ float s_part[kWaves][D];
  const int b = u / a.Hkv;
  const int kv = u % a.Hkv;
  const int r = a.Hq / a.Hkv;
  const int rpu = r * a.Nq;
  const int row0 = (b * a.Hq + kv * r) * a.Nq;  // the unit's rows are consecutive
  const int NS = a.n_c + a.n_g;
  const int Tb = route_seq_len(a, b);
  if (Tb <= 0) return;  // no keys: every row of the unit routes to nothing
  const int cf = max(0, Tb - a.Nq) / a.C;  // first chunk holding one of the newest Nq keys
  const int cl = (Tb - 1) / a.C;
  const size_t bkv = static_cast<size_t>(u);
  const float* cm = a.chunk_mean + bkv * a.n_c * D;
  const float* gm = a.group_mean + bkv * a.n_g * D;
  // The unit's query rows (at most kPreQ) are read first, before anything the
  // item waits for, and staged in LDS once.
  __shared__ float s_q[kPreQ][D];
  const bool pre_q = rpu <= kPreQ;
  uint4 qr0, qr1;
  q_issue<TQ, D>(a, row0, pre_q ? rpu : 0, qr0, qr1);
  // Refreshed groups: with enough items, each has an item of its own (items
  // 1..nfg), which sums the group's keys itself (the same bits as item 0's
  // chunk summary) and scores it; item 0 then scores only the refreshed chunks
  // below the newest, and its chunk summaries are needed only as outputs.
  const int g0 = cf * a.gpc;
  const int nfg = min((cl + 1) * a.gpc, (Tb + a.G - 1) / a.G) - g0;
  const bool own_items = s.items >= nfg + 2;
  const int first_old = own_items ? nfg + 1 : 1;
  constexpr int EPL = Elem<TQ>::kPer16;
  if (m == 0) {
    for (int c = cf; c <= cl; ++c) {
      chunk_summary<TQ, D, kWaves>(
          static_cast<const TQ*>(a.K), a.kv, b, a.Hkv, kv, a.T, Tb, a.C, a.G, c, s_part,
          [&](int g, int col, const float (&sum)[EPL], int count) {
            const float inv = 1.f / static_cast<float>(count);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
              s_fr[rowroute::kFreshChunks + g - cf * a.gpc][col + e] = sum[e] * inv;
          },
          [&](int d, float sum, int count) {
            s_fr[c - cf][d] = sum / static_cast<float>(count);
          });
      __syncthreads();
    }
    const int nfc = cl - cf;                  // scored chunks: cf .. cl - 1
    const int n = nfc + (own_items ? 0 : nfg);
    if (n > 0) {
      if (pre_q) {
        q_stage<TQ, D>(a, rpu, qr0, qr1, s_q);
        __syncthreads();
      }
      // (one LDS base, so that these reads are known to be LDS reads and do
      // not wait for outstanding global memory operations)
      score_block<TQ, D>(
          a, row0, rpu, n,
          [&](int i) { return &s_fr[i < nfc ? i : rowroute::kFreshChunks + i - nfc][0]; },
          [&](int i) { return i < nfc ? cf + i : a.n_c + g0 + i - nfc; }, s.scores, NS,
          pre_q ? s_q : nullptr);
    }
  } else if (m < first_old) {
    // refreshed group g, summed by wave 0 (row 0 of s_fr as scratch)
    const int g = g0 + m - 1;
    if (threadIdx.x < kWave) {
      float acc[EPL];
      const int count = group_key_sum<TQ, D>(static_cast<const TQ*>(a.K), a.kv, b, a.Hkv, kv,
                                             a.T, Tb, a.G, g, acc);
      const float inv = 1.f / static_cast<float>(count);
      constexpr int LPR = D / EPL;
      if (lane_id() < LPR) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_fr[0][lane_id() * EPL + e] = acc[e] * inv;
      }
    }
    if (pre_q) q_stage<TQ, D>(a, rpu, qr0, qr1, s_q);
    __syncthreads();
    score_block<TQ, D>(
        a, row0, rpu, 1, [&](int) { return &s_fr[0][0]; }, [&](int) { return a.n_c + g; },
        s.scores, NS, pre_q ? s_q : nullptr);
  } else {
    // the older summaries: chunks [0, cf), then groups [0, cf * gpc)
    const int n_old = cf * (1 + a.gpc);
    const int n_items = s.items - first_old;
    const int per = (n_old + n_items - 1) / n_items;
    const int j0 = (m - first_old) * per;
    const int j1 = min(n_old, j0 + per);
    if (j0 < j1) {
      score_block<TQ, D>(
          a, row0, rpu, j1 - j0,
          [&](int i) {
            const int j = j0 + i;
            return j < cf ? cm + static_cast<size_t>(j) * D : gm + static_cast<size_t>(j - cf) * D;
          },
          [&](int i) {
            const int j = j0 + i;
            return j < cf ? j : a.n_c + j - cf;
          },
          s.scores, NS, pre_q ? s_q : nullptr, pre_q, qr0, qr1);
    }
  }
}

// Item 0 of unit u, at the end of its workgroup's work: the refreshed
// summaries go out from LDS (nothing in the launch reads them, so their stores
// need not hold up the workgroup's attention part).
template <int D>
__device__ __forceinline__ void write_refreshed(const RouteArgs& a, int u, const FreshRows<D>& s_fr) {
  const int b = u / a.Hkv;
  const int Tb = route_seq_len(a, b);
  if (Tb <= 0) return;
  const int cf = max(0, Tb - a.Nq) / a.C;
  const int cl = (Tb - 1) / a.C;
  const int nfc = cl - cf + 1;
  const int g0 = cf * a.gpc;
  const int nfg = min((cl + 1) * a.gpc, (Tb + a.G - 1) / a.G) - g0;
  float* cm_w = const_cast<float*>(a.chunk_mean) + (static_cast<size_t>(u) * a.n_c + cf) * D;
  float* gm_w = const_cast<float*>(a.group_mean) + (static_cast<size_t>(u) * a.n_g + g0) * D;
  for (int t = static_cast<int>(threadIdx.x); t < (nfc + nfg) * D; t += kThreads) {
    const int i = t / D, d = t % D;
    if (i < nfc) {
      cm_w[t] = s_fr[i][d];
    } else {
      gm_w[t - nfc * D] = s_fr[rowroute::kFreshChunks + i - nfc][d];
    }
  }
}

// Dynamic LDS of the step: the row's scores [n_c + n_g] | kept chunks [cap] |
// the row's group ids [k_g].
inline size_t step_lds_bytes(const RouteArgs& a) {
  const int cap = kept_capacity(a);
  return static_cast<size_t>(a.n_c + a.n_g + cap + a.k_g) * 4;
}

template <typename T, int D, int E>
__global__ __launch_bounds__(kThreads) void decode_kernel(RouteArgs ra, AttendArgs aa,
                                                          StepArgs st) {
  extern __shared__ float s_dyn[];
  __shared__ bool s_ok;
  const int bid = static_cast<int>(blockIdx.x);
  const int U = ra.B * ra.Hkv;
  HGA_PHASE(0);
  // The workspace's status word, loaded first and read only after the scoring
  // item: non-zero if a wait of an earlier step on this workspace gave up.
  const int32_t status0 = load_shared_i32(aa.status);
  __shared__ FreshRows<D> s_fr;
  if (bid < U * st.items) score_item<T, D>(ra, st, bid % U, bid / U, s_fr);
  HGA_PHASE(1);
  const int rows = ra.B * ra.Hq * ra.Nq;
  if (bid >= rows * st.n_splits) {
    if (bid < U) write_refreshed<D>(ra, bid, s_fr);
    return;
  }

  // ---- this workgroup's attention item: row, split
  const int row = bid / st.n_splits;
  const int split = bid % st.n_splits;
  const int i = row % ra.Nq;
  const int b = row / ra.Nq / ra.Hq;
  const int Tb = route_seq_len(ra, b);
  const int p = Tb - ra.Nq + i;
  const int NS = ra.n_c + ra.n_g;
  int32_t* words = st.scores + static_cast<size_t>(row) * NS;

  const int cap = kept_capacity(ra);
  float* s_cs = s_dyn;               // chunk scores [n_c]
  float* s_gs = s_cs + ra.n_c;       // group scores [n_g]
  int* s_kept = reinterpret_cast<int*>(s_gs + ra.n_g);
  int* s_ids = s_kept + cap;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int L = p >= 0 ? p / ra.C : -1;
  // The row's score words: every word the scoring writes for the row (a
  // superset of chunks 0..L and groups 0..p/G, so that each word is known to
  // have landed before it is zeroed again). A polling thread loads its words
  // with all loads in flight and reloads the ones still zero (not written yet)
  // until none is (bounded: the row is poisoned if not), decoding them into
  // LDS. Chunk words [c0, c1) and group words [g0, g1), spread over the nthr
  // threads numbered tid.
  auto poll = [&](int c0, int c1, int g0, int g1, int tid, int nthr) {
    const int nc = c1 - c0, total = nc + g1 - g0;
    bool arrived = true;
    for (int base = 0; base < total; base += 8 * nthr) {
      int32_t v[8];
      unsigned pending = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int idx = base + k * nthr + tid;
        v[k] = 1;
        if (idx < total) v[k] = load_shared_i32(words + (idx < nc ? c0 + idx : ra.n_c + g0 + idx - nc));
        pending |= static_cast<unsigned>(v[k] == 0) << k;
      }
      for (int it = 0; pending != 0u && it < (1 << 20); ++it) {
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int idx = base + k * nthr + tid;
          if ((pending >> k) & 1u)
            v[k] = load_shared_i32(words + (idx < nc ? c0 + idx : ra.n_c + g0 + idx - nc));
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) pending &= ~(static_cast<unsigned>(v[k] != 0) << k);
      }
      arrived = arrived && pending == 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int idx = base + k * nthr + tid;
        if (idx < total) s_dyn[idx < nc ? c0 + idx : ra.n_c + g0 + idx - nc] = handoff_float(v[k]);
      }
    }
    if (!arrived) {
      s_ok = false;
      store_shared_i32(aa.status, kStatusTimedOut);
    }
  };
  // Level 1 (wave 0): chunk 0, chunk L and the k_chunk best between.
  auto level1 = [&]() -> int {
    if (L + 1 <= ra.k_c + 2) {
      for (int t = lane; t <= L; t += kWave) s_kept[t] = t;
      wave_lds_sync();
      return L + 1;
    }
    // chunks 1..L-1 compete; the chosen ones land in s_kept[1..k_c] directly
    if (ra.k_c > 0)
      rowroute::wave_select_ids_fit<E>(
          L - 1, ra.k_c,
          [&](int t, int& id) {
            id = 1 + t;
            return s_cs[1 + t];
          },
          s_kept + 1, nullptr);
    if (lane == 0) {
      s_kept[0] = 0;
      s_kept[ra.k_c + 1] = L;
    }
    wave_lds_sync();
    return ra.k_c + 2;
  };

  // The older words come from the other scoring items, the refreshed ones
  // (chunks cf.., groups cf * gpc..) from the refreshing items, which finish
  // last. Level 1 needs only chunks 1..L-1, so when those are all older
  // chunks (the early case: every decode row), wave 0 polls the older chunk
  // words alone (a few scoring items write them) and selects while the other
  // waves poll the group words and the refreshed ones.
  int n1 = 0, n2 = 0, cf = 0;
  if (Tb > 0) {
    written_range(ra, Tb, n1, n2);
    cf = max(0, Tb - ra.Nq) / ra.C;
  }
  const int gf = min(cf * ra.gpc, n2);
  const bool early = p >= 0 && L - 1 < cf;
  // After a wait that gave up, late stores may have left words in the zero
  // region: a step on such a workspace reads no word and poisons its rows
  // (until the caller resets the workspace).
  const bool stale = status0 != 0;
  if (threadIdx.x == 0) s_ok = !stale;
  __syncthreads();
  int n_kept = 0;
  if (early) {
    if (wave == 0) {
      if (!stale) {
        poll(0, cf, 0, 0, lane, kWave);
        wave_lds_sync();
        HGA_PHASE(2);
        n_kept = level1();
      }
      HGA_PHASE(10);
    } else if (!stale) {
      poll(0, 0, 0, gf, threadIdx.x - kWave, kThreads - kWave);
      poll(cf, n1, gf, n2, threadIdx.x - kWave, kThreads - kWave);
    }
    __syncthreads();
  } else {
    if (!stale) {
      poll(0, cf, 0, gf, threadIdx.x, kThreads);
      poll(cf, n1, gf, n2, threadIdx.x, kThreads);
    }
    __syncthreads();
    HGA_PHASE(2);
    if (wave == 0 && p >= 0 && !stale) n_kept = level1();
  }
  HGA_PHASE(3);
  const bool ok = s_ok;
  if (wave == 0) {
    int got = 0;
    if (!ok) n_kept = 0;  // a poisoned row routes to nothing
    // Candidate t of level 2 is group s_kept[t / gpc] * gpc + t % gpc (kept
    // chunks ascending, so the candidates ascend too).
    const int gpc = ra.gpc;
    // t / gpc as a multiply-high by ceil(2^32 / gpc): exact for t * gpc < 2^32
    // (here t < 4096 items, gpc <= 512), and no branch
    // (ceil(2^32 / gpc) from a 32-bit division: floor((2^32 - 1) / gpc) + 1 is
    // the same number for every gpc >= 1, and a 64-bit division is a long
    // scalar sequence on the critical path)
    const uint64_t magic = static_cast<uint64_t>(0xFFFFFFFFu / static_cast<uint32_t>(gpc)) + 1u;
    auto cand = [&](int t) {
      const int k = static_cast<int>((static_cast<uint64_t>(t) * magic) >> 32);
      return s_kept[k] * gpc + (t - k * gpc);
    };
    int32_t* gout = split == 0 ? ra.group_idx + static_cast<size_t>(row) * ra.k_g : nullptr;
    if (p >= 0 && ok) {
      // level 2: the groups of the kept chunks that start at or before p; the
      // invalid ones are the last kept chunk's (chunk L's) groups after p. The
      // chosen group ids go to s_ids (and split 0's to group_idx) directly.
      const int n_valid = (n_kept - 1) * gpc + min(gpc, p / ra.G - L * gpc + 1);
      got = rowroute::wave_select_ids<E>(
          n_valid, ra.k_g,
          [&](int t, int& id) {
            id = cand(t);
            return s_gs[id];
          },
          s_ids, gout);
      HGA_PHASE(11);
    }
    for (int t = got + lane; t < ra.k_g; t += kWave) {
      s_ids[t] = -1;
      if (gout) gout[t] = -1;
    }
    if (split == 0 && ra.chunk_idx) {
      for (int t = lane; t < ra.k_c + 2; t += kWave)
        ra.chunk_idx[static_cast<size_t>(row) * (ra.k_c + 2) + t] = t < n_kept ? s_kept[t] : -1;
    }
  }
  __syncthreads();
  HGA_PHASE(4);
  // Every split of the row has read the row's scores once all have counted
  // themselves in: the finishing workgroup then zeroes every word the scoring
  // wrote for the row (each one it saw arrive).
  // (n1, n2: written_range's counts, taken before the polls)
  auto zero_row = [&]() {
    for (int t = static_cast<int>(threadIdx.x); t < n1 + n2; t += kThreads)
      store_shared_i32(words + (t < n1 ? t : ra.n_c + t - n1), 0);
  };
  attend_body<T, D, kWaves, true, decltype(zero_row), true>(aa, st.groups_per_wave, st.n_splits,
                                                           0, bid, s_ids, !ok, zero_row);
  if (bid < U) write_refreshed<D>(ra, bid, s_fr);
  HGA_PHASE(9);
}

// Scoring items per unit: as many as the grid holds (at least two: the refresh
// and the older summaries). U * items <= the CU count (U <= CUs / 2).
int step_items(int64_t units, int cus) {
  return static_cast<int>(std::max<int64_t>(2, cus / units));
}

template <typename T, int D>
hipError_t launch_td(const RouteArgs& ra, const AttendArgs& aa, const StepArgs& st,
                     hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(ra.B) * ra.Hq * ra.Nq;
  const int64_t U = static_cast<int64_t>(ra.B) * ra.Hkv;
  const int64_t n = std::max<int64_t>(U * st.items, rows * st.n_splits);
  const dim3 grid(static_cast<unsigned>(n));
  const size_t lds = step_lds_bytes(ra);
  switch (select_regs(ra)) {
#define HGA_DECODE_CASE(EV)                                                                    \
  case EV: {                                                                                   \
    if (lds > 65536) {                                                                         \
      const hipError_t e = hipFuncSetAttribute(                                                \
          reinterpret_cast<const void*>(&decode_kernel<T, D, EV>),                             \
          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));                  \
      if (e != hipSuccess) return e;                                                           \
    }                                                                                          \
    hipLaunchKernelGGL((decode_kernel<T, D, EV>), grid, dim3(kThreads), lds, stream, ra, aa, st); \
    break;                                                                                     \
  }
    HGA_DECODE_CASE(1)
    HGA_DECODE_CASE(2)
    HGA_DECODE_CASE(3)
    HGA_DECODE_CASE(4)
    HGA_DECODE_CASE(5)
    HGA_DECODE_CASE(6)
    HGA_DECODE_CASE(8)
    HGA_DECODE_CASE(16)
    HGA_DECODE_CASE(32)
    HGA_DECODE_CASE(64)
#undef HGA_DECODE_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Static LDS of decode_kernel (bound): the refresh's rows and the attention's.
size_t step_static_lds(int64_t D) {
  const int fresh_rows = rowroute::kFreshChunks * (1 + rowroute::kFreshMaxGpc) + kWaves + kPreQ;
  return static_cast<size_t>(fresh_rows * D + 2 * kWaves + kWaves * D +
                             kAttendMaxSplits * (D + 2)) * 4 + 64;
}

}  // namespace

// Where the step's hand-off words sit in the zero-at-rest region: the rows'
// score words after the counters, then the splits' partials.
struct StepWords {
  size_t scores, partials, end;
};
static StepWords step_words(int64_t rows, int64_t NS, int n_splits, int64_t D) {
  StepWords w{};
  w.scores = kCounterBytes;
  w.partials = (w.scores + static_cast<size_t>(rows * NS) * 4 + 255) / 256 * 256;
  w.end = w.partials + (n_splits > 1 ? static_cast<size_t>(rows * n_splits * (D + 2)) * 4 : 0);
  return w;
}

AttendPlan plan_decode_attend(int64_t rows, int64_t D, int k_g, int cus) {
  // The fewest groups per wave (8 waves per workgroup) that keep one
  // workgroup per (row, split) within one per CU.
  const int W = kWaves;
  int gpw = 1;
  while (gpw < k_g &&
         (rows * ((k_g + W * gpw - 1) / (W * gpw)) > cus ||
          (k_g + W * gpw - 1) / (W * gpw) > kAttendMaxSplits))
    gpw *= 2;
  AttendPlan pl{};
  pl.groups_per_wave = gpw;
  pl.n_splits = (k_g + W * gpw - 1) / (W * gpw);
  // the partials are hand-off words in the zero-at-rest region (step_words)
  pl.off_counters = 0;
  pl.off_partials = 0;
  pl.bytes = kZeroBytes;
  return pl;
}

bool decode_step_one_launch(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t T, int64_t D,
                            int C, int G, int k_c, int k_g, int cus) {
  const int64_t rows = B * Hq * Nq, units = B * Hkv;
  if (cus < 2 || 2 * units > cus) return false;
  if (Nq > C || C / G > rowroute::kFreshMaxGpc) return false;  // the refresh's LDS rows
  const AttendPlan plan = plan_decode_attend(rows, D, k_g, cus);
  if (rows * plan.n_splits > cus) return false;
  const int64_t n_c = (T + C - 1) / C, n_g = (T + G - 1) / G;
  // the score and partial words live in the workspace's zero-at-rest region
  if (step_words(rows, n_c + n_g, plan.n_splits, D).end > kStatusOffset) return false;
  const int64_t cap = std::min<int64_t>(k_c + 2, n_c);
  const size_t lds = static_cast<size_t>(n_c + n_g + cap + k_g) * 4;
  return lds + step_static_lds(D) <= 160 * 1024;
}

size_t decode_step_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t D, int k_g) {
  return plan_decode_attend(B * Hq * Nq, D, k_g, kPlanCus).bytes;
}

hipError_t launch_decode_step(const RouteArgs& ra, const AttendArgs& aa, const AttendPlan& plan,
                              int dtype, void* workspace, int cus, hipStream_t stream) {
  const StepWords w = step_words(static_cast<int64_t>(ra.B) * ra.Hq * ra.Nq, ra.n_c + ra.n_g,
                                 plan.n_splits, ra.D);
  char* ws = static_cast<char*>(workspace);
  StepArgs st{};
  st.scores = reinterpret_cast<int32_t*>(ws + w.scores);
  AttendArgs a2 = aa;
  a2.partials = reinterpret_cast<float*>(ws + w.partials);
  a2.status = reinterpret_cast<int32_t*>(ws + kStatusOffset);
  st.items = step_items(static_cast<int64_t>(ra.B) * ra.Hkv, cus);
  st.n_splits = plan.n_splits;
  st.groups_per_wave = plan.groups_per_wave;
  if (dtype == kF32)
    return ra.D == 64 ? launch_td<float, 64>(ra, a2, st, stream)
                      : launch_td<float, 128>(ra, a2, st, stream);
  return ra.D == 64 ? launch_td<uint16_t, 64>(ra, a2, st, stream)
                    : launch_td<uint16_t, 128>(ra, a2, st, stream);
}

}  // namespace hga

#ifdef HGA_PHASE_STAMPS
// Sets the phase-stamp buffer of the one-launch decode step (16 x 8 bytes per
// workgroup), or none with NULL. Phase-stamp builds only.
extern "C" int hga_debug_phase_stamps(void* buffer) {
  unsigned long long* p = static_cast<unsigned long long*>(buffer);
  return hipMemcpyToSymbol(HIP_SYMBOL(g_hga_phase_stamps), &p, sizeof(p)) == hipSuccess ? 0 : -7;
}
#endif

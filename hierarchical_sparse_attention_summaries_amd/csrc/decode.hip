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
// sequence holds Tb > 0 keys: chunks [0, n_chunks), groups [0, n_groups).
__device__ __forceinline__ void written_range(const RouteArgs& a, int Tb, int& n_chunks,
                                              int& n_groups) {
  const int cl = (Tb - 1) / a.C;
  n_chunks = cl + 1;
  n_groups = min((cl + 1) * a.gpc, (Tb + a.G - 1) / a.G);
}

// Scores summary rows i in [0, n) (row_ptr(i): D floats, all of one pointer
// kind) against query rows row0 .. row0 + nq - 1: the score of query row j and
// summary row i goes to scores[(row0 + j) * NS + col_of(i)] as a score word. Lane l of wave w
// holds dims [(l % LPR) * 8, +8) of summary rows w * RPS + l / LPR + k * kStride;
// the dot product is the row route's, in the same order, so both give the same
// bits.
template <typename TQ, int D, typename RowPtr, typename ColOf>
__device__ __forceinline__ void score_block(const RouteArgs& a, int row0, int nq, int n,
                                            RowPtr row_ptr, ColOf col_of, int32_t* scores,
                                            int NS) {
  constexpr int LPR = D / 8;
  constexpr int RPS = kWave / LPR;
  constexpr int kStride = kWaves * RPS;
  constexpr int NB = 2;  // summary rows per lane per pass
  constexpr int QB = 8;  // query rows per pass
  const int lane = lane_id();
  const int col = (lane % LPR) * 8;
  const int first = (threadIdx.x / kWave) * RPS + lane / LPR;
  for (int base = 0; base < n; base += NB * kStride) {
    float4 v0[NB], v1[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = base + first + j * kStride;
      if (i < n) {
        const float* src = row_ptr(i) + col;
        v0[j] = *reinterpret_cast<const float4*>(src);
        v1[j] = *reinterpret_cast<const float4*>(src + 4);
      } else {
        v0[j] = v1[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    for (int qb = 0; qb < nq; qb += QB) {
      float q[QB][8];
#pragma unroll
      for (int r = 0; r < QB; ++r) {
        if (qb + r < nq) {
          const size_t off = static_cast<size_t>(row0 + qb + r) * D + col;
          if constexpr (sizeof(TQ) == 4) {
            float x0[4], x1[4];
            widen(ld16(static_cast<const float*>(a.Q) + off), x0);
            widen(ld16(static_cast<const float*>(a.Q) + off + 4), x1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              q[r][e] = x0[e] * a.scale;
              q[r][4 + e] = x1[e] * a.scale;
            }
          } else {
            widen(ld16(static_cast<const uint16_t*>(a.Q) + off), q[r]);
#pragma unroll
            for (int e = 0; e < 8; ++e) q[r][e] *= a.scale;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) q[r][e] = 0.f;
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

// Scoring item m of unit u (see the top of the file).
template <typename TQ, int D>
__device__ __forceinline__ void score_item(const RouteArgs& a, const StepArgs& s, int u, int m) {
  __shared__ float s_fc[rowroute::kFreshChunks][D];
  __shared__ float s_fg[rowroute::kFreshChunks * rowroute::kFreshMaxGpc][D];
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
  if (m == 0) {
    constexpr int EPL = Elem<TQ>::kPer16;
    float* cm_w = const_cast<float*>(cm);
    float* gm_w = const_cast<float*>(gm);
    for (int c = cf; c <= cl; ++c) {
      chunk_summary<TQ, D, kWaves>(
          static_cast<const TQ*>(a.K), a.kv, b, a.Hkv, kv, a.T, Tb, a.C, a.G, c, s_part,
          [&](int g, int col, const float (&sum)[EPL], int count) {
            const float inv = 1.f / static_cast<float>(count);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              const float v = sum[e] * inv;
              gm_w[static_cast<size_t>(g) * D + col + e] = v;
              s_fg[g - cf * a.gpc][col + e] = v;
            }
          },
          [&](int d, float sum, int count) {
            const float v = sum / static_cast<float>(count);
            cm_w[static_cast<size_t>(c) * D + d] = v;
            s_fc[c - cf][d] = v;
          });
      __syncthreads();
    }
    const int nfc = cl - cf + 1;
    const int g0 = cf * a.gpc;
    const int nfg = min((cl + 1) * a.gpc, (Tb + a.G - 1) / a.G) - g0;
    score_block<TQ, D>(
        a, row0, rpu, nfc + nfg,
        [&](int i) { return i < nfc ? &s_fc[i][0] : &s_fg[i - nfc][0]; },
        [&](int i) { return i < nfc ? cf + i : a.n_c + g0 + i - nfc; }, s.scores, NS);
  } else {
    // the older summaries: chunks [0, cf), then groups [0, cf * gpc)
    const int n_old = cf * (1 + a.gpc);
    const int per = (n_old + s.items - 2) / (s.items - 1);
    const int j0 = (m - 1) * per;
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
          s.scores, NS);
    }
  }
}

// Dynamic LDS of the step: the row's scores [n_c + n_g] | kept chunks [cap] |
// candidate group ids [cap * gpc] | chosen [max(k_c, k_g)] | the row's ids [k_g].
inline size_t step_lds_bytes(const RouteArgs& a) {
  const int cap = kept_capacity(a);
  return static_cast<size_t>(a.n_c + a.n_g + cap + cap * a.gpc + max(a.k_c, a.k_g) + a.k_g) * 4;
}

template <typename T, int D, int E>
__global__ __launch_bounds__(kThreads) void decode_kernel(RouteArgs ra, AttendArgs aa,
                                                          StepArgs st) {
  extern __shared__ float s_dyn[];
  __shared__ bool s_ok;
  const int bid = static_cast<int>(blockIdx.x);
  const int U = ra.B * ra.Hkv;
  if (bid < U * st.items) score_item<T, D>(ra, st, bid % U, bid / U);
  const int rows = ra.B * ra.Hq * ra.Nq;
  if (bid >= rows * st.n_splits) return;

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
  int* s_gid = s_kept + cap;
  int* s_pick = s_gid + cap * ra.gpc;
  int* s_ids = s_pick + max(ra.k_c, ra.k_g);
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int L = p >= 0 ? p / ra.C : -1;
  if (threadIdx.x == 0) s_ok = true;
  __syncthreads();
  if (Tb > 0) {
    // Every word the scoring writes for the row (a superset of chunks 0..L and
    // groups 0..p/G, so that each word is known to have landed before it is
    // zeroed again). Every thread loads its words with all loads in flight and
    // reloads the ones still zero (not written yet) until none is (bounded:
    // the row is poisoned if not).
    int n1, n2;
    written_range(ra, Tb, n1, n2);
    bool ok = true;
    for (int base = 0; base < n1 + n2; base += 8 * kThreads) {
      int32_t v[8];
      unsigned pending = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int idx = base + k * kThreads + static_cast<int>(threadIdx.x);
        v[k] = 1;
        if (idx < n1 + n2) v[k] = load_shared_i32(words + (idx < n1 ? idx : ra.n_c + idx - n1));
        pending |= static_cast<unsigned>(v[k] == 0) << k;
      }
      for (int it = 0; pending != 0u && it < (1 << 20); ++it) {
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int idx = base + k * kThreads + static_cast<int>(threadIdx.x);
          if ((pending >> k) & 1u) v[k] = load_shared_i32(words + (idx < n1 ? idx : ra.n_c + idx - n1));
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) pending &= ~(static_cast<unsigned>(v[k] != 0) << k);
      }
      ok = ok && pending == 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int idx = base + k * kThreads + static_cast<int>(threadIdx.x);
        if (idx < n1 + n2) s_dyn[idx < n1 ? idx : ra.n_c + idx - n1] = handoff_float(v[k]);
      }
    }
    if (!ok) s_ok = false;
  }
  __syncthreads();
  const bool ok = s_ok;
  if (wave == 0) {
    int n_kept = 0;
    int got = 0;
    if (p >= 0 && ok) {
      // level 1: chunk 0, chunk L and the k_chunk best between
      if (L + 1 <= ra.k_c + 2) {
        n_kept = L + 1;
        for (int t = lane; t < n_kept; t += kWave) s_kept[t] = t;
      } else {
        n_kept = ra.k_c + 2;
        const int gc = ra.k_c > 0 ? rowroute::wave_select<E>(
                                        L - 1, ra.k_c, [&](int t) { return s_cs[1 + t]; }, s_pick)
                                  : 0;
        wave_lds_sync();
        for (int t = lane; t < gc; t += kWave) s_kept[1 + t] = 1 + s_pick[t];
        if (lane == 0) {
          s_kept[0] = 0;
          s_kept[n_kept - 1] = L;
        }
      }
      wave_lds_sync();
      // level 2: the groups of the kept chunks that start at or before p;
      // invalid candidates sit only at the end of the list (last kept chunk)
      const int n_cand = n_kept * ra.gpc;
      int n_valid = 0;
      for (int t = lane; t < n_cand; t += kWave) {
        const int g = s_kept[t / ra.gpc] * ra.gpc + t % ra.gpc;
        s_gid[t] = g;
        n_valid += (g < ra.n_g && static_cast<int64_t>(g) * ra.G <= p) ? 1 : 0;
      }
      n_valid = static_cast<int>(wave_add(static_cast<uint32_t>(n_valid)));
      wave_lds_sync();
      got = rowroute::wave_select<E>(n_valid, ra.k_g, [&](int t) { return s_gs[s_gid[t]]; },
                                     s_pick);
      wave_lds_sync();
    }
    for (int t = lane; t < ra.k_g; t += kWave) {
      const int g = t < got ? s_gid[s_pick[t]] : -1;
      s_ids[t] = g;
      if (split == 0) ra.group_idx[static_cast<size_t>(row) * ra.k_g + t] = g;
    }
    if (split == 0 && ra.chunk_idx) {
      for (int t = lane; t < ra.k_c + 2; t += kWave)
        ra.chunk_idx[static_cast<size_t>(row) * (ra.k_c + 2) + t] = t < n_kept ? s_kept[t] : -1;
    }
  }
  __syncthreads();
  // Every split of the row has read the row's scores once all have counted
  // themselves in: the finishing workgroup then zeroes every word the scoring
  // wrote for the row (each one it saw arrive).
  auto zero_row = [&]() {
    if (Tb <= 0) return;
    int n_chunks, n_groups;
    written_range(ra, Tb, n_chunks, n_groups);
    for (int t = static_cast<int>(threadIdx.x); t < n_chunks + n_groups; t += kThreads)
      store_shared_i32(words + (t < n_chunks ? t : ra.n_c + t - n_chunks), 0);
  };
  attend_body<T, D, false, kWaves, true, decltype(zero_row), true>(
      aa, st.groups_per_wave, st.n_splits, 0, bid, nullptr, s_ids, !ok, zero_row);
}

// Scoring items per unit: as many as the grid holds (at least two: the refresh
// and the older summaries). U * items <= the CU count (U <= CUs / 2).
int step_items(int64_t units) {
  const int64_t cus = device_cu_count();
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
  const int fresh_rows = rowroute::kFreshChunks + rowroute::kFreshChunks * rowroute::kFreshMaxGpc +
                         kWaves;
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

AttendPlan plan_decode_attend(int64_t rows, int64_t D, int k_g) {
  // The fewest groups per wave (8 waves per workgroup) that keep one
  // workgroup per (row, split) within one per CU.
  const int W = kWaves;
  int gpw = 1;
  while (gpw < k_g &&
         (rows * ((k_g + W * gpw - 1) / (W * gpw)) > device_cu_count() ||
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
                            int C, int G, int k_c, int k_g) {
  const int64_t cus = device_cu_count();
  const int64_t rows = B * Hq * Nq, units = B * Hkv;
  if (2 * units > cus) return false;
  if (Nq > C || C / G > rowroute::kFreshMaxGpc) return false;  // the refresh's LDS rows
  const AttendPlan plan = plan_decode_attend(rows, D, k_g);
  if (rows * plan.n_splits > cus) return false;
  const int64_t n_c = (T + C - 1) / C, n_g = (T + G - 1) / G;
  // the score and partial words live in the workspace's zero-at-rest region
  if (step_words(rows, n_c + n_g, plan.n_splits, D).end > kZeroBytes) return false;
  const int64_t cap = std::min<int64_t>(k_c + 2, n_c);
  const size_t lds = static_cast<size_t>(n_c + n_g + cap + cap * (C / G) + std::max(k_c, k_g) + k_g) * 4;
  return lds + step_static_lds(D) <= 160 * 1024;
}

size_t decode_step_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t D, int k_g) {
  return plan_decode_attend(B * Hq * Nq, D, k_g).bytes;
}

hipError_t launch_decode_step(const RouteArgs& ra, const AttendArgs& aa, const AttendPlan& plan,
                              int dtype, void* workspace, hipStream_t stream) {
  const StepWords w = step_words(static_cast<int64_t>(ra.B) * ra.Hq * ra.Nq, ra.n_c + ra.n_g,
                                 plan.n_splits, ra.D);
  char* ws = static_cast<char*>(workspace);
  StepArgs st{};
  st.scores = reinterpret_cast<int32_t*>(ws + w.scores);
  AttendArgs a2 = aa;
  a2.partials = reinterpret_cast<float*>(ws + w.partials);
  st.items = step_items(static_cast<int64_t>(ra.B) * ra.Hkv);
  st.n_splits = plan.n_splits;
  st.groups_per_wave = plan.groups_per_wave;
  if (dtype == kF32)
    return ra.D == 64 ? launch_td<float, 64>(ra, a2, st, stream)
                      : launch_td<float, 128>(ra, a2, st, stream);
  return ra.D == 64 ? launch_td<uint16_t, 64>(ra, a2, st, stream)
                    : launch_td<uint16_t, 128>(ra, a2, st, stream);
}

}  // namespace hga

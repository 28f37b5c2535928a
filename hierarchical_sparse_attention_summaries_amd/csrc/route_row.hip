// Step 2 of HGA (abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709), one workgroup per query row: the two levels exactly as stated.
// The workgroup scores the query against the summaries of chunks 0..L (L = the
// query's own chunk), keeps chunk 0, chunk L and the k_chunk best of the chunks
// between, then gathers and scores only the groups of the kept chunks and keeps
// the k_group best of them. Everything between the two summary reads stays in
// LDS, so a row costs two memory round trips and no workgroup waits for or
// hands data to another. Used when few query rows are routed at once (small
// decode batches), where latency, not bytes, sets the time.
#include "hga_device.h"
#include "hga_internal.h"
#include "hga_select.h"
#include "hga_summary.h"

namespace hga {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kBatch = 8;  // wave-steps of summary loads in flight per lane

// Scores summary rows src(0..n-1) for query q: row i -> out[i] (LDS).
// 16 lanes per row (8 dims each, D = 128) or 8 lanes (D = 64).
template <int D, typename RowPtr>
__device__ __forceinline__ void score_rows(const float (&q)[8], int n, RowPtr row_ptr, float* out) {
  constexpr int LPR = D / 8;
  constexpr int RPS = kWave / LPR;
  constexpr int kStride = kWaves * RPS;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int sub = lane / LPR;
  const int col = (lane % LPR) * 8;
  for (int base0 = wave * RPS; base0 < n; base0 += kBatch * kStride) {
    float4 v0[kBatch], v1[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = base0 + j * kStride + sub;
      if (i < n) {
        const float* src = row_ptr(i) + col;
        v0[j] = *reinterpret_cast<const float4*>(src);
        v1[j] = *reinterpret_cast<const float4*>(src + 4);
      } else {
        v0[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        v1[j] = v0[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = base0 + j * kStride + sub;
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
}

// Top-k of n keys held in LDS (`score(i)` gives item i's float score), by one
// wave; writes the chosen item ids ascending to out[0..k) and returns how many.
template <int E, typename ScoreOf>
__device__ __forceinline__ int wave_select(int n, int k, ScoreOf score, int* out) {
  const int lane = lane_id();
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * kWave + lane;
    key[e] = i < n ? order_key(score(i)) : 0u;
  }
  uint32_t chosen = 0;
  if (n <= k) {
#pragma unroll
    for (int e = 0; e < E; ++e) chosen |= static_cast<uint32_t>(key[e] != 0u) << e;
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

constexpr int kFreshChunks = 2;   // chunks a refresh of <= C newest keys can touch
constexpr int kFreshMaxGpc = 16;  // groups per chunk the refresh keeps in LDS

template <typename TQ, int D, int E, bool FRESH>
__global__ __launch_bounds__(kThreads) void route_row_kernel(RouteArgs a) {
  extern __shared__ float s_dyn[];
  // LDS: chunk scores [n_c] | candidate scores [cap * gpc] | kept chunks [cap] | chosen [max]
  const int cap = kept_capacity(a);
  float* s_cs = s_dyn;
  float* s_gs = s_cs + a.n_c;
  int* s_kept = reinterpret_cast<int*>(s_gs + cap * a.gpc);
  int* s_pick = s_kept + cap;
  __shared__ int s_n_kept;

  // Workgroups are dealt to the 8 XCDs round-robin by index; give every query
  // row of one (sequence, KV head) the same residue mod 8, so that the rows
  // sharing chunk summaries share an L2. Indices past the last unit idle.
  const int rpu = (a.Hq / a.Hkv) * a.Nq;  // rows per (sequence, KV head)
  const int xcd = blockIdx.x % 8;
  const int k = blockIdx.x / 8;
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

  // Refresh: the chunks holding the sequence's newest Nq keys are recomputed
  // from K (same bits as the summaries kernel), written out, and scored from
  // LDS. Every row of this (sequence, KV head) writes the same values.
  int cf = 1, cl = 0;  // refreshed chunk range (empty unless FRESH)
  __shared__ float s_fc[FRESH ? kFreshChunks : 1][D];
  __shared__ float s_fg[FRESH ? kFreshChunks * kFreshMaxGpc : 1][D];
  __shared__ float s_part[FRESH ? kWaves : 1][D];
  if constexpr (FRESH) {
    constexpr int EPL = Elem<TQ>::kPer16;
    const int Tb = route_seq_len(a, b);
    cf = max(0, Tb - a.Nq) / a.C;
    cl = (Tb - 1) / a.C;
    float* cm_w = const_cast<float*>(cm);
    float* gm_w = const_cast<float*>(gm);
    for (int c = cf; c <= cl; ++c) {
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
  auto chunk_row = [&](int c) -> const float* {
    if (FRESH && c >= cf && c <= cl) return &s_fc[c - cf][0];
    return cm + static_cast<size_t>(c) * D;
  };

  // Level 1: chunks 0..L.
  score_rows<D>(q, L + 1, chunk_row, s_cs);
  __syncthreads();
  if (wave == 0) {
    int n_kept;
    if (L + 1 <= a.k_c + 2) {
      n_kept = L + 1;
      for (int t = lane; t < n_kept; t += kWave) s_kept[t] = t;
    } else {
      n_kept = a.k_c + 2;
      const int got = a.k_c > 0 ? wave_select<E>(L - 1, a.k_c, [&](int t) { return s_cs[1 + t]; },
                                                 s_pick)
                                : 0;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int t = lane; t < got; t += kWave) s_kept[1 + t] = 1 + s_pick[t];
      if (lane == 0) {
        s_kept[0] = 0;
        s_kept[n_kept - 1] = L;
      }
    }
    if (lane == 0) s_n_kept = n_kept;
  }
  __syncthreads();
  const int n_kept = s_n_kept;
  if (a.chunk_idx) {
    for (int t = threadIdx.x; t < a.k_c + 2; t += kThreads)
      a.chunk_idx[static_cast<size_t>(row) * (a.k_c + 2) + t] = t < n_kept ? s_kept[t] : -1;
  }

  // Level 2: the groups of the kept chunks that start at or before p.
  const int n_cand = n_kept * a.gpc;
  auto gid = [&](int t) { return s_kept[t / a.gpc] * a.gpc + t % a.gpc; };
  auto valid = [&](int t) {
    const int g = gid(t);
    return g < a.n_g && static_cast<int64_t>(g) * a.G <= p;
  };
  score_rows<D>(q, n_cand, [&](int t) -> const float* {
    const int g = gid(t);
    if (FRESH && g / a.gpc >= cf && g / a.gpc <= cl) return &s_fg[g - cf * a.gpc][0];
    return gm + static_cast<size_t>(g < a.n_g ? g : 0) * D;
  }, s_gs);
  __syncthreads();
  if (wave == 0) {
    // Invalid candidates sit only in the last kept chunk (after p or past the
    // end), i.e. at the end of the list: select among the valid prefix.
    int n_valid = 0;
    for (int t = lane; t < n_cand; t += kWave) n_valid += valid(t) ? 1 : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) n_valid += __shfl_xor(n_valid, m, kWave);
    const int got = wave_select<E>(n_valid, a.k_g, [&](int t) { return s_gs[t]; }, s_pick);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    int32_t* out = a.group_idx + static_cast<size_t>(row) * a.k_g;
    for (int t = lane; t < a.k_g; t += kWave) out[t] = t < got ? gid(s_pick[t]) : -1;
  }
}

template <typename TQ, int D, bool FRESH>
hipError_t launch_td(const RouteArgs& a, int e_sel, size_t lds, hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(a.B) * a.Hkv;
  const int64_t rpu = static_cast<int64_t>(a.Hq / a.Hkv) * a.Nq;
  const dim3 grid(static_cast<unsigned>(8 * ((units + 7) / 8) * rpu));
  switch (e_sel) {
#define HGA_ROW_CASE(EV)                                                                         \
  case EV:                                                                                       \
    hipLaunchKernelGGL((route_row_kernel<TQ, D, EV, FRESH>), grid, dim3(kThreads), lds, stream, a); \
    break;
    HGA_ROW_CASE(1)
    HGA_ROW_CASE(2)
    HGA_ROW_CASE(3)
    HGA_ROW_CASE(4)
    HGA_ROW_CASE(5)
    HGA_ROW_CASE(6)
    HGA_ROW_CASE(8)
    HGA_ROW_CASE(16)
    HGA_ROW_CASE(32)
    default:
      hipLaunchKernelGGL((route_row_kernel<TQ, D, 64, FRESH>), grid, dim3(kThreads), lds, stream, a);
      break;
#undef HGA_ROW_CASE
  }
  return hipGetLastError();
}

}  // namespace

bool use_row_route(int64_t B, int64_t Hq, int64_t Nq) { return B * Hq * Nq <= 1024; }

bool row_route_can_refresh(int64_t Nq, int C, int G) {
  return Nq <= C && C / G <= kFreshMaxGpc;
}

hipError_t launch_route_rows(const RouteArgs& a, int dtype, hipStream_t stream) {
  const int cap = kept_capacity(a);
  const size_t lds = (static_cast<size_t>(a.n_c) + static_cast<size_t>(cap) * a.gpc) * 4 +
                     static_cast<size_t>(cap) * 4 + static_cast<size_t>(kMaxSelectItems) * 4;
  const int e_sel = select_regs(a);
  if (a.K) {
    if (dtype == kF32)
      return a.D == 64 ? launch_td<float, 64, true>(a, e_sel, lds, stream)
                       : launch_td<float, 128, true>(a, e_sel, lds, stream);
    return a.D == 64 ? launch_td<uint16_t, 64, true>(a, e_sel, lds, stream)
                     : launch_td<uint16_t, 128, true>(a, e_sel, lds, stream);
  }
  if (dtype == kF32)
    return a.D == 64 ? launch_td<float, 64, false>(a, e_sel, lds, stream)
                     : launch_td<float, 128, false>(a, e_sel, lds, stream);
  return a.D == 64 ? launch_td<uint16_t, 64, false>(a, e_sel, lds, stream)
                   : launch_td<uint16_t, 128, false>(a, e_sel, lds, stream);
}

}  // namespace hga

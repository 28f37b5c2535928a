// Step 2 of HGA (abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709): two-level routing per query head. Chunks are retrieved by the
// score of their mean key; inside the retrieved chunks only the best groups are
// kept. The first chunk and the query's own chunk are always retrieved.
//
// One launch. Workgroups of a (sequence, KV head, block of <= 16 query rows)
// each score a slice of chunks and the groups of those chunks for every query
// row of the block (the r query heads that share the KV head read the same
// summary bytes once). The slices' scores go to the workspace; the last
// workgroup of the block to finish (an atomic arrival count, nobody waits)
// runs the selection: one wave per query row does a bitwise radix top-k of the
// chunks with ballots, then lists the kept chunks' groups and runs the same
// top-k on them.
//
// Why all groups are scored: with GQA the r query heads of a KV head each
// examine (k_chunk + 2) * chunk/group candidate groups; at the budgets used with
// this method (k_chunk ~ n_chunks/8, r = 8) those candidate sets together cover
// every group of the head, so one dense pass over the group summaries moves no
// more bytes than gathering each head's candidates, and it needs no second
// launch between the chunk and the group level. Only candidates of the kept
// chunks can be selected, so the routed sets are those of the two-level rule.
#include "hga_device.h"
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;  // one query row per wave in the selection
constexpr int kMaxRows = 16;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Selection for one query row, run by one whole wave.
template <int E>
__device__ __forceinline__ void select_row(const RouteArgs& a, int row, int p, int* s_kept) {
  const int lane = lane_id();
  const int L = p / a.C;  // the query's own chunk
  const float* cs = a.chunk_scores + static_cast<size_t>(row) * a.n_c;
  const float* gs = a.group_scores + static_cast<size_t>(row) * a.n_g;
  int n_kept;
  if (L + 1 <= a.k_c + 2) {
    n_kept = L + 1;
    for (int t = lane; t < n_kept; t += kWave) s_kept[t] = t;
  } else {
    n_kept = a.k_c + 2;
    if (lane == 0) {
      s_kept[0] = 0;
      s_kept[n_kept - 1] = L;
    }
    if (a.k_c > 0) {
      // candidates: chunks 1 .. L-1, item t <-> chunk 1 + t
      uint32_t key[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int t = e * kWave + lane;
        key[e] = t < L - 1 ? order_key(load_shared(cs + 1 + t)) : 0u;
      }
      const uint32_t chosen = wave_top_k<E>(key, a.k_c);
      int before = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool c = (chosen >> e) & 1u;
        const uint64_t m = ballot(c);
        if (c) s_kept[1 + before + bits_below(m)] = 1 + e * kWave + lane;
        before += __popcll(m);
      }
    }
  }
  wave_lds_sync();
  if (a.chunk_idx) {
    int32_t* out = a.chunk_idx + static_cast<size_t>(row) * (a.k_c + 2);
    for (int t = lane; t < a.k_c + 2; t += kWave) out[t] = t < n_kept ? s_kept[t] : -1;
  }
  // candidate groups of the kept chunks, in ascending group order
  const int n_items = n_kept * a.gpc;
  uint32_t key[E];
  int gid[E];
  int n_valid = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int t = e * kWave + lane;
    bool valid = false;
    int g = -1;
    if (t < n_items) {
      g = s_kept[t / a.gpc] * a.gpc + t % a.gpc;
      valid = g < a.n_g && static_cast<int64_t>(g) * a.G <= p;
    }
    gid[e] = g;
    key[e] = valid ? order_key(load_shared(gs + g)) : 0u;
    n_valid += __popcll(ballot(valid));
  }
  uint32_t chosen = 0;
  if (n_valid <= a.k_g) {
#pragma unroll
    for (int e = 0; e < E; ++e) chosen |= static_cast<uint32_t>(key[e] != 0u) << e;
  } else {
    chosen = wave_top_k<E>(key, a.k_g);
  }
  int32_t* out = a.group_idx + static_cast<size_t>(row) * a.k_g;
  int before = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool c = (chosen >> e) & 1u;
    const uint64_t m = ballot(c);
    if (c) out[before + bits_below(m)] = gid[e];
    before += __popcll(m);
  }
  for (int t = before + lane; t < a.k_g; t += kWave) out[t] = -1;
  wave_lds_sync();  // s_kept is reused by this wave's next row
}

template <typename TQ, int D, int RM>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a, int n_qblocks,
                                                         int chunks_per_split, int n_splits,
                                                         int e_sel) {
  constexpr int DPL = 8;          // summary dims per lane (two 16-byte fp32 loads)
  constexpr int LPR = D / DPL;    // lanes per summary row
  constexpr int RPS = kWave / LPR;
  extern __shared__ int s_kept_all[];
  __shared__ bool s_last;

  const int unit = blockIdx.x / n_splits;
  const int split = blockIdx.x % n_splits;
  const int qb = unit % n_qblocks;
  const int bkv = unit / n_qblocks;
  const int kv = bkv % a.Hkv;
  const int b = bkv / a.Hkv;
  const int r = a.Hq / a.Hkv;
  const int rows_here = min(kMaxRows, r * a.Nq - qb * kMaxRows);  // <= RM by the plan
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // Row rho of this block is query i = (qb*16 + rho) / r of head kv*r + (qb*16 + rho) % r.
  auto row_of = [&](int rho) {
    const int gr = qb * kMaxRows + rho;
    const int h = kv * r + gr % r;
    const int i = gr / r;
    return (b * a.Hq + h) * a.Nq + i;
  };

  // Each lane keeps, for every query row of the block, the 8 query dims it
  // multiplies (loaded straight into registers, scaled).
  const int sub = lane / LPR;
  const int col = (lane % LPR) * DPL;
  float qr[RM][DPL];
#pragma unroll
  for (int rho = 0; rho < RM; ++rho) {
    if (rho < rows_here) {
      const size_t off = static_cast<size_t>(row_of(rho)) * D + col;
      if constexpr (sizeof(TQ) == 4) {
        float x0[4], x1[4];
        widen(ld16(static_cast<const float*>(a.Q) + off), x0);
        widen(ld16(static_cast<const float*>(a.Q) + off + 4), x1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qr[rho][e] = x0[e] * a.scale;
          qr[rho][4 + e] = x1[e] * a.scale;
        }
      } else {
        float x[8];
        widen(ld16(static_cast<const uint16_t*>(a.Q) + off), x);
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[rho][e] = x[e] * a.scale;
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) qr[rho][e] = 0.f;
    }
  }

  const int c_lo = split * chunks_per_split;
  const int c_hi = min(c_lo + chunks_per_split, a.n_c);
  const int n_ch = c_hi - c_lo;
  const int n_items = n_ch * (1 + a.gpc);  // chunk rows first, then their groups
  const float* cm = a.chunk_mean + static_cast<size_t>(b * a.Hkv + kv) * a.n_c * D;
  const float* gm = a.group_mean + static_cast<size_t>(b * a.Hkv + kv) * a.n_g * D;

  // Summary rows of this workgroup, kBatch wave-steps of loads in flight at a time.
  constexpr int kBatch = 4;
  constexpr int kStride = kWaves * RPS;
  for (int base0 = wave * RPS; base0 < n_items; base0 += kBatch * kStride) {
    float sv[kBatch][DPL];
    int dst_col[kBatch];
    bool valid[kBatch], is_chunk[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int item = base0 + j * kStride + sub;
      is_chunk[j] = item < n_ch;
      dst_col[j] = is_chunk[j] ? c_lo + item : c_lo * a.gpc + (item - n_ch);
      valid[j] = item < n_items && (is_chunk[j] || dst_col[j] < a.n_g);
      if (valid[j]) {
        const float* src = (is_chunk[j] ? cm : gm) + static_cast<size_t>(dst_col[j]) * D + col;
        const float4 v0 = *reinterpret_cast<const float4*>(src);
        const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
        sv[j][0] = v0.x; sv[j][1] = v0.y; sv[j][2] = v0.z; sv[j][3] = v0.w;
        sv[j][4] = v1.x; sv[j][5] = v1.y; sv[j][6] = v1.z; sv[j][7] = v1.w;
      } else {
#pragma unroll
        for (int e = 0; e < DPL; ++e) sv[j][e] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (base0 + j * kStride >= n_items) break;  // wave-uniform
      float* dst_base = is_chunk[j] ? a.chunk_scores : a.group_scores;
      const int dst_stride = is_chunk[j] ? a.n_c : a.n_g;
#pragma unroll
      for (int rho = 0; rho < RM; ++rho) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) d = fmaf(qr[rho][e], sv[j][e], d);
        d = group_sum<LPR>(d);
        if (valid[j] && rho < rows_here && (lane % LPR) == (rho % LPR))
          store_shared(dst_base + static_cast<size_t>(row_of(rho)) * dst_stride + dst_col[j], d);
      }
    }
  }

  if (!arrive_last(a.counters + unit, static_cast<unsigned>(n_splits), &s_last)) return;

  int* s_kept = s_kept_all + wave * (a.k_c + 2 > a.n_c ? a.n_c : a.k_c + 2);
  for (int rho = wave; rho < rows_here; rho += kWaves) {
    const int row = row_of(rho);
    const int p = a.T - a.Nq + (qb * kMaxRows + rho) / r;
    switch (e_sel) {
      case 1: select_row<1>(a, row, p, s_kept); break;
      case 2: select_row<2>(a, row, p, s_kept); break;
      case 3: select_row<3>(a, row, p, s_kept); break;
      case 4: select_row<4>(a, row, p, s_kept); break;
      case 5: select_row<5>(a, row, p, s_kept); break;
      case 6: select_row<6>(a, row, p, s_kept); break;
      case 8: select_row<8>(a, row, p, s_kept); break;
      case 16: select_row<16>(a, row, p, s_kept); break;
      case 32: select_row<32>(a, row, p, s_kept); break;
      default: select_row<64>(a, row, p, s_kept); break;
    }
  }
}

template <typename TQ, int D>
hipError_t launch_rm(const RouteArgs& a, const RoutePlan& plan, int rm, int e_sel,
                     size_t lds, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv *
                                                plan.n_qblocks * plan.n_splits);
  if (rm == 8) {
    hipLaunchKernelGGL((route_kernel<TQ, D, 8>), dim3(blocks), dim3(kThreads), lds, stream, a,
                       plan.n_qblocks, plan.chunks_per_split, plan.n_splits, e_sel);
  } else {
    hipLaunchKernelGGL((route_kernel<TQ, D, 16>), dim3(blocks), dim3(kThreads), lds, stream, a,
                       plan.n_qblocks, plan.chunks_per_split, plan.n_splits, e_sel);
  }
  return hipGetLastError();
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

RoutePlan plan_route(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t T, int C, int G,
                     int k_c, int k_g) {
  (void)k_g;
  (void)k_c;
  RoutePlan pl{};
  const int64_t r = Hq / Hkv;
  const int64_t n_c = (T + C - 1) / C;
  const int64_t n_g = (T + G - 1) / G;
  pl.q_per_block = kMaxRows;
  pl.n_qblocks = static_cast<int>((r * Nq + kMaxRows - 1) / kMaxRows);
  // Few workgroups per arrival counter (they bump it one after another), but
  // at most 16 chunks (16 * (1 + chunk/group) summary rows) per workgroup.
  const int64_t units = B * Hkv * pl.n_qblocks;
  const int64_t target = static_cast<int64_t>(device_cu_count()) / 2;
  int64_t splits = (target + units - 1) / units;
  const int64_t min_splits = (n_c + 15) / 16;
  if (splits < min_splits) splits = min_splits;
  if (splits < 1) splits = 1;
  if (splits > n_c) splits = n_c;
  pl.chunks_per_split = static_cast<int>((n_c + splits - 1) / splits);
  pl.n_splits = static_cast<int>((n_c + pl.chunks_per_split - 1) / pl.chunks_per_split);
  const int64_t rows = B * Hq * Nq;
  pl.off_counters = 0;
  pl.off_chunk_scores = align_up(static_cast<size_t>(units) * sizeof(unsigned), 256);
  pl.off_group_scores = align_up(pl.off_chunk_scores + static_cast<size_t>(rows * n_c) * 4, 256);
  pl.bytes = align_up(pl.off_group_scores + static_cast<size_t>(rows * n_g) * 4, 256);
  return pl;
}

hipError_t launch_route(const RouteArgs& a, int dtype, const RoutePlan& plan, hipStream_t stream) {
  const int r = a.Hq / a.Hkv;
  const int max_rows = r * a.Nq < kMaxRows ? r * a.Nq : kMaxRows;
  const int rm = max_rows <= 8 ? 8 : 16;
  const int kept = a.k_c + 2 > a.n_c ? a.n_c : a.k_c + 2;
  const int items = (a.n_c - 2 > kept * a.gpc) ? a.n_c - 2 : kept * a.gpc;
  // registers per lane for the selection keys: the smallest variant that fits
  const int need = (items + kWave - 1) / kWave;
  int e_sel = 64;
  for (int e : {1, 2, 3, 4, 5, 6, 8, 16, 32, 64}) {
    if (e >= need) {
      e_sel = e;
      break;
    }
  }
  const int kept_per_wave = a.k_c + 2 > a.n_c ? a.n_c : a.k_c + 2;
  const size_t lds = static_cast<size_t>(kWaves) * kept_per_wave * sizeof(int);
  if (dtype == kF32)
    return a.D == 64 ? launch_rm<float, 64>(a, plan, rm, e_sel, lds, stream)
                     : launch_rm<float, 128>(a, plan, rm, e_sel, lds, stream);
  return a.D == 64 ? launch_rm<uint16_t, 64>(a, plan, rm, e_sel, lds, stream)
                   : launch_rm<uint16_t, 128>(a, plan, rm, e_sel, lds, stream);
}

}  // namespace hga

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
// runs the selection: one wave per query row does a radix top-k of the chunks
// with ballots (two bits per step), then lists the kept chunks' groups and
// runs the same top-k on them.
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
#include "hga_select.h"

namespace hga {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;  // one query row per wave in the selection
constexpr int kMaxRows = 16;

template <typename TQ, int D, int RM>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a, int n_qblocks,
                                                         int chunks_per_split, int n_splits,
                                                         int e_sel, int kept_cap, int unit_base) {
  constexpr int DPL = 8;          // summary dims per lane (two 16-byte fp32 loads)
  constexpr int LPR = D / DPL;    // lanes per summary row
  constexpr int RPS = kWave / LPR;
  // Dynamic LDS: first the score staging [RM][items] (phase 1), then, after
  // the arrival barrier, the per-wave kept-chunk lists (selection).
  extern __shared__ int s_dyn[];
  float* s_stage = reinterpret_cast<float*>(s_dyn);
  __shared__ bool s_last;

  const int unit = unit_base + static_cast<int>(blockIdx.x) / n_splits;
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
      const int item = base0 + j * kStride + sub;
#pragma unroll
      for (int rho = 0; rho < RM; ++rho) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) d = fmaf(qr[rho][e], sv[j][e], d);
        d = group_sum<LPR>(d);
        if (valid[j] && (lane % LPR) == (rho % LPR)) s_stage[rho * n_items + item] = d;
      }
    }
  }
  __syncthreads();
  // Each query row's scores of this slice are contiguous in the workspace:
  // chunk scores [c_lo, c_hi), group scores from c_lo * gpc. Write them out
  // with consecutive lanes on consecutive columns.
  {
    const int n_grp = min(n_ch * a.gpc, a.n_g - c_lo * a.gpc);
    const int per_row = n_ch + n_grp;
    for (int idx = threadIdx.x; idx < rows_here * per_row; idx += kThreads) {
      const int rho = idx / per_row;
      const int it = idx % per_row;
      const size_t row = static_cast<size_t>(row_of(rho));
      float* dst = it < n_ch ? a.chunk_scores + row * a.n_c + c_lo + it
                             : a.group_scores + row * a.n_g + c_lo * a.gpc + (it - n_ch);
      store_shared(dst, s_stage[rho * n_items + it]);
    }
  }

  if (!arrive_last(a.counters + (unit - unit_base), static_cast<unsigned>(n_splits), &s_last))
    return;

  int* s_kept = s_dyn + wave * kept_cap;
  for (int rho = wave; rho < rows_here; rho += kWaves) {
    const int row = row_of(rho);
    const int p = route_seq_len(a, b) - a.Nq + (qb * kMaxRows + rho) / r;
    select_row_e(e_sel, a, row, p, s_kept);
  }
}

template <typename TQ, int D>
hipError_t launch_rm(const RouteArgs& a, const RoutePlan& plan, int rm, int e_sel,
                     int kept_cap, hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(a.B) * a.Hkv * plan.n_qblocks;
  const size_t stage = static_cast<size_t>(rm) * plan.chunks_per_split * (1 + a.gpc) * sizeof(float);
  const size_t kept = static_cast<size_t>(kWaves) * kept_cap * sizeof(int);
  const size_t lds = stage > kept ? stage : kept;
  // Slices of at most kMaxCounters units, one counter each; stream order lets
  // a slice reuse the counters the previous one left at zero.
  for (int64_t base = 0; base < units; base += kMaxCounters) {
    const int64_t n = units - base < kMaxCounters ? units - base : kMaxCounters;
    const dim3 grid(static_cast<unsigned>(n * plan.n_splits));
    if (rm == 8) {
      hipLaunchKernelGGL((route_kernel<TQ, D, 8>), grid, dim3(kThreads), lds, stream, a,
                         plan.n_qblocks, plan.chunks_per_split, plan.n_splits, e_sel, kept_cap,
                         static_cast<int>(base));
    } else {
      hipLaunchKernelGGL((route_kernel<TQ, D, 16>), grid, dim3(kThreads), lds, stream, a,
                         plan.n_qblocks, plan.chunks_per_split, plan.n_splits, e_sel, kept_cap,
                         static_cast<int>(base));
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
  // About one round of workgroups over the chip (a later round would wait for
  // a whole earlier one, and the selection runs after the last), few
  // workgroups per arrival counter (they bump it one after another), and at
  // most 768 summary rows per workgroup (their scores for 16 query rows are
  // staged in 48 KiB of LDS).
  const int64_t units = B * Hkv * pl.n_qblocks;
  const int64_t target = static_cast<int64_t>(kPlanCus);
  int64_t splits = (target + units - 1) / units;
  const int64_t gpc = C / G;
  int64_t max_cps = 768 / (1 + gpc);
  if (max_cps < 1) max_cps = 1;
  const int64_t min_splits = (n_c + max_cps - 1) / max_cps;
  if (splits < min_splits) splits = min_splits;
  if (splits < 1) splits = 1;
  if (splits > n_c) splits = n_c;
  pl.chunks_per_split = static_cast<int>((n_c + splits - 1) / splits);
  pl.n_splits = static_cast<int>((n_c + pl.chunks_per_split - 1) / pl.chunks_per_split);
  const int64_t rows = B * Hq * Nq;
  pl.off_counters = 0;
  pl.off_chunk_scores = kZeroBytes;
  pl.off_group_scores = align_up(pl.off_chunk_scores + static_cast<size_t>(rows * n_c) * 4, 256);
  pl.bytes = align_up(pl.off_group_scores + static_cast<size_t>(rows * n_g) * 4, 256);
  pl.off_split = 0;
  if (r * Nq >= 64) {  // many query rows per KV head: room for the MFMA operand copies
    pl.off_split = pl.bytes;
    pl.bytes = align_up(pl.off_split + static_cast<size_t>(B * Hkv * (n_c + n_g) * 128) * 4, 256);
  }
  return pl;
}

hipError_t launch_route(const RouteArgs& a, int dtype, const RoutePlan& plan, hipStream_t stream) {
  const int r = a.Hq / a.Hkv;
  const int max_rows = r * a.Nq < kMaxRows ? r * a.Nq : kMaxRows;
  const int rm = max_rows <= 8 ? 8 : 16;
  const int e_sel = select_regs(a);
  const int kept_cap = kept_capacity(a);
  if (dtype == kF32)
    return a.D == 64 ? launch_rm<float, 64>(a, plan, rm, e_sel, kept_cap, stream)
                     : launch_rm<float, 128>(a, plan, rm, e_sel, kept_cap, stream);
  return a.D == 64 ? launch_rm<uint16_t, 64>(a, plan, rm, e_sel, kept_cap, stream)
                   : launch_rm<uint16_t, 128>(a, plan, rm, e_sel, kept_cap, stream);
}

}  // namespace hga

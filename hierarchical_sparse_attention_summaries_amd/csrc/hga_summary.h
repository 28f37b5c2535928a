// Summaries of one chunk by one 8-wave workgroup (step 1 of HGA, abstract of
// "Hierarchical Global Attention (HGA)", arXiv 2606.30709: the mean post-RoPE
// key of each group and of the chunk). Shared by the summaries kernel and the
// decode route that refreshes the newest chunk itself, so both produce the
// same bits: the same rows go to the same lanes and are summed in the same
// order.
#pragma once

#include "hga_device.h"
#include "hga_internal.h"

namespace hga {

// One wave's loads of up to kRows consecutive key rows (16 bytes per lane,
// 8 in flight): lane l takes dims [(l % LPR) * EPL, +EPL) of rows
// u * RPL + l / LPR. Issuing and adding are separate so that a caller can
// keep the loads in flight across other work.
template <typename TK, int D>
struct KeyRowLoads {
  static constexpr int EPL = Elem<TK>::kPer16;  // elements per lane per load
  static constexpr int LPR = D / EPL;           // lanes per key row
  static constexpr int RPL = kWave / LPR;       // rows per load instruction
  static constexpr int UNROLL = 8;
  static constexpr int kRows = RPL * UNROLL;
  uint4 raw[UNROLL];

  // rows [base, base + kRows) of the n rows at Kg (rows past n read as zero)
  __device__ __forceinline__ void issue(const TK* __restrict__ Kg, int base, int n) {
    const int lane = lane_id();
    const int col = (lane % LPR) * EPL;
    const int sub = lane / LPR;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int t = base + u * RPL + sub;
      raw[u] = t < n ? ld16(Kg + static_cast<size_t>(t) * D + col) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) raw[u] = make_uint4(0, 0, 0, 0);
  }
  // acc += the rows, in row-slot order
  __device__ __forceinline__ void add_to(float (&acc)[EPL]) const {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float x[EPL];
      widen(raw[u], x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += x[e];
    }
  }
};

// Where group g of (b, kv) starts in K (its rows are consecutive) and how many
// of its rows lie below Tb; the offset is negative where no page holds it.
__device__ __forceinline__ int64_t group_rows(const KvLayout& L, int b, int Hkv, int kv, int T,
                                              int D, int Tb, int G, int g, int* n) {
  const int t0 = g * G;
  *n = min(t0 + G, Tb) - t0;
  return kv_offset(L, b, Hkv, kv, T, D, t0);
}

// The sum of group g's keys (rows [g * G, min(g * G + G, Tb)) of (b, kv)), by
// one wave: KeyRowLoads passes with fp32 accumulation, then a fold over the
// rows; lane l ends with dims [(l % LPR) * EPL, +EPL) of the sum (every row
// added in a fixed order, so every caller gets the same bits). Returns the
// group's row count.
template <typename TK, int D>
__device__ __forceinline__ int group_key_sum(const TK* __restrict__ K, const KvLayout& L, int b,
                                             int Hkv, int kv, int T, int Tb, int G, int g,
                                             float (&acc)[Elem<TK>::kPer16]) {
  using R = KeyRowLoads<TK, D>;
  int n;
  const int64_t off = group_rows(L, b, Hkv, kv, T, D, Tb, G, g, &n);
#pragma unroll
  for (int e = 0; e < R::EPL; ++e) acc[e] = 0.f;
  if (off >= 0) {
    for (int base = 0; base < n; base += R::kRows) {
      R r;
      r.issue(K + off, base, n);
      r.add_to(acc);
    }
  }
#pragma unroll
  for (int e = 0; e < R::EPL; ++e) acc[e] = across_rows_sum<R::LPR>(acc[e]);
  return n;
}

// Wave w sums groups g_first + w, g_first + w + WAVES, ... of chunk c of
// (b, kv) with group_key_sum. put_group(g, col, sums, count) runs on the
// lanes holding columns col .. col+EPL-1 of group g (sums not yet divided);
// the waves' group sums meet in s_part, and after a workgroup barrier
// put_chunk(d, chunk_sum, count) runs on threads d < D.
template <typename TK, int D, int WAVES, typename PutGroup, typename PutChunk>
__device__ __forceinline__ void chunk_summary(const TK* __restrict__ K, const KvLayout& L, int b,
                                              int Hkv, int kv, int T, int Tb, int C, int G, int c,
                                              float (*s_part)[D], PutGroup put_group,
                                              PutChunk put_chunk) {
  constexpr int EPL = Elem<TK>::kPer16;   // elements per lane per load
  constexpr int LPR = D / EPL;            // lanes per key row
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int col = (lane % LPR) * EPL;
  const int sub = lane / LPR;
  const int gpc = C / G;
  const int g_first = c * gpc;
  const int g_end = min(g_first + gpc, (Tb + G - 1) / G);

  float csum[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) csum[e] = 0.f;
  for (int g = g_first + wave; g < g_end; g += WAVES) {
    float acc[EPL];
    const int count = group_key_sum<TK, D>(K, L, b, Hkv, kv, T, Tb, G, g, acc);
    if (sub == 0) put_group(g, col, acc, count);
#pragma unroll
    for (int e = 0; e < EPL; ++e) csum[e] += acc[e];
  }
  if (sub == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_part[wave][col + e] = csum[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += s_part[w][threadIdx.x];
    put_chunk(static_cast<int>(threadIdx.x), s, min(C, Tb - c * C));
  }
}

}  // namespace hga

// Step 1 of HGA (abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709): compact summaries of the post-RoPE keys. A summary is the mean
// key of a group (G tokens) or of a chunk (C = gpc * G tokens).
//
// One workgroup per (sequence, KV head, chunk). Keys come from a dense
// [B, Hkv, T, D] cache or from pages through a block table; a group's rows are
// always consecutive, and sequences may hold fewer than T keys. Each wave
// streams whole groups
// with 16-byte coalesced loads (a row of D elements is spread over D*size/16
// lanes, so one wave-wide load covers 64*16/(D*size) rows), accumulates in fp32
// registers, folds the rows of the group with cross-lane adds, writes the group
// mean, and keeps the group sum for the chunk; the eight waves' chunk partials
// meet in LDS. HBM-bound: every key is read exactly once.
#include "hga_device.h"
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kThreads = 512;  // 8 waves: one group of a 256-token chunk each
constexpr int kWaves = kThreads / kWave;

template <typename TK, int D>
__global__ __launch_bounds__(kThreads) void summaries_kernel(
    const TK* __restrict__ K, KvLayout L, float* __restrict__ chunk_mean,
    float* __restrict__ group_mean, int Hkv, int T, int C, int G, int n_c, int n_g, int c_begin,
    int n_chunks_here, int newest) {
  constexpr int EPL = Elem<TK>::kPer16;   // elements per lane per load
  constexpr int LPR = D / EPL;            // lanes per key row
  constexpr int RPL = kWave / LPR;        // rows per wave-wide load
  constexpr int UNROLL = 8;               // loads in flight per lane

  __shared__ float s_part[kWaves][D];

  const int bh = blockIdx.x / n_chunks_here;
  const int b = bh / Hkv;
  const int kv = bh % Hkv;
  const int Tb = seq_len_of(L, b, T);
  const int c0 = newest > 0 ? max(0, Tb - newest) / C : c_begin;
  const int c = c0 + blockIdx.x % n_chunks_here;
  if (c * C >= Tb) return;  // beyond this sequence's keys: nothing to summarise
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int col = (lane % LPR) * EPL;
  const int sub = lane / LPR;             // row slot within a load

  const int gpc = C / G;
  const int g_first = c * gpc;
  const int g_end = min(g_first + gpc, (Tb + G - 1) / G);

  float csum[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) csum[e] = 0.f;

  for (int g = g_first + wave; g < g_end; g += kWaves) {
    const int t0 = g * G;
    const int t1 = min(t0 + G, Tb);
    const int64_t off = kv_offset(L, b, Hkv, kv, T, D, t0);  // the group's rows are consecutive
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    if (off >= 0) {
      const TK* Kg = K + off;
      for (int base = 0; base < t1 - t0; base += RPL * UNROLL) {
        uint4 raw[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int t = base + u * RPL + sub;
          raw[u] = t < t1 - t0 ? ld16(Kg + static_cast<size_t>(t) * D + col) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          float x[EPL];
          widen(raw[u], x);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] += x[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = across_rows_sum<LPR>(acc[e]);
    const float inv = 1.f / static_cast<float>(t1 - t0);
    if (sub == 0) {
      float* dst = group_mean + (static_cast<size_t>(bh) * n_g + g) * D + col;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dst[e] = acc[e] * inv;
    }
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
    for (int w = 0; w < kWaves; ++w) s += s_part[w][threadIdx.x];
    const int t0 = c * C;
    const int t1 = min(t0 + C, Tb);
    chunk_mean[(static_cast<size_t>(bh) * n_c + c) * D + threadIdx.x] =
        s / static_cast<float>(t1 - t0);
  }
}

template <typename TK, int D>
hipError_t launch_t(const void* K, const KvLayout& L, float* cm, float* gm, int64_t BH, int Hkv,
                    int T, int C, int G, int c_begin, int n_here, int newest, hipStream_t stream) {
  const int n_c = (T + C - 1) / C;
  const int n_g = (T + G - 1) / G;
  const int64_t blocks = BH * n_here;
  hipLaunchKernelGGL((summaries_kernel<TK, D>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream, static_cast<const TK*>(K), L, cm, gm, Hkv, T, C, G,
                     n_c, n_g, c_begin, n_here, newest);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_summaries(const void* K, int dtype, const KvLayout& L, int64_t B, int64_t Hkv,
                            int64_t D, int64_t T, int C, int G, int c_begin, int n_chunks,
                            int64_t newest, float* chunk_mean, float* group_mean,
                            hipStream_t stream) {
  const int t = static_cast<int>(T);
  const int64_t BH = B * Hkv;
  const int h = static_cast<int>(Hkv);
  const int nw = static_cast<int>(newest);
  if (dtype == kF32) {
    return D == 64 ? launch_t<float, 64>(K, L, chunk_mean, group_mean, BH, h, t, C, G, c_begin, n_chunks, nw, stream)
                   : launch_t<float, 128>(K, L, chunk_mean, group_mean, BH, h, t, C, G, c_begin, n_chunks, nw, stream);
  }
  return D == 64 ? launch_t<uint16_t, 64>(K, L, chunk_mean, group_mean, BH, h, t, C, G, c_begin, n_chunks, nw, stream)
                 : launch_t<uint16_t, 128>(K, L, chunk_mean, group_mean, BH, h, t, C, G, c_begin, n_chunks, nw, stream);
}

}  // namespace hga

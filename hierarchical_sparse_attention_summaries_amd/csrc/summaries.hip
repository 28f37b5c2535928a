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
#include "hga_summary.h"

namespace hga {
namespace {

constexpr int kThreads = 512;  // 8 waves: one group of a 256-token chunk each
constexpr int kWaves = kThreads / kWave;

template <typename TK, int D>
__global__ __launch_bounds__(kThreads) void summaries_kernel(
    const TK* __restrict__ K, KvLayout L, float* __restrict__ chunk_mean,
    float* __restrict__ group_mean, int Hkv, int T, int C, int G, int n_c, int n_g, int c_begin,
    int n_chunks_here, int newest) {
  constexpr int EPL = Elem<TK>::kPer16;
  __shared__ float s_part[kWaves][D];

  const int bh = blockIdx.x / n_chunks_here;
  const int b = bh / Hkv;
  const int kv = bh % Hkv;
  const int Tb = seq_len_of(L, b, T);
  const int c0 = newest > 0 ? max(0, Tb - newest) / C : c_begin;
  const int c = c0 + blockIdx.x % n_chunks_here;
  if (c * C >= Tb) return;  // beyond this sequence's keys: nothing to summarise
  chunk_summary<TK, D, kWaves>(
      K, L, b, Hkv, kv, T, Tb, C, G, c, s_part,
      [&](int g, int col, const float (&sum)[EPL], int count) {
        const float inv = 1.f / static_cast<float>(count);
        float* dst = group_mean + (static_cast<size_t>(bh) * n_g + g) * D + col;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[e] = sum[e] * inv;
      },
      [&](int d, float sum, int count) {
        chunk_mean[(static_cast<size_t>(bh) * n_c + c) * D + d] = sum / static_cast<float>(count);
      });
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

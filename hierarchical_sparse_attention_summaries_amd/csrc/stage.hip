// Attention over K/V that the device reads slowly (pinned host memory): the
// host-memory tier of HGA (abstract of "Hierarchical Global Attention (HGA)",
// arXiv 2606.30709: the full K/V need not live in device memory; only the
// routed tokens are fetched). The r*Nq query rows of one (sequence, KV head)
// route to overlapping groups, so each routed group is copied once into a
// device pool and attention then reads the pool:
//   mark:   a bit per (sequence, KV head, group) routed by any of its rows;
//   assign: per (sequence, KV head), the marked groups get consecutive pool
//           pages (ascending group order) -> block table and page -> group;
//   gather: one workgroup per pool page copies the group's G keys and values.
// Attention then runs as B*Hkv sequences of one KV head each over the pool as
// a paged cache, with the same arithmetic in the same order as on the source.
#include <hip/hip_runtime.h>

#include "hga_device.h"
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kStageThreads = 256;

__global__ __launch_bounds__(kStageThreads) void clear_kernel(uint32_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kStageThreads + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// One thread per group-id entry: mark its (sequence, KV head, group).
__global__ __launch_bounds__(kStageThreads) void mark_kernel(const int32_t* group_idx,
                                                             int64_t entries, int k_g, int Hq,
                                                             int Nq, int r, int n_g, int words,
                                                             uint32_t* marks) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kStageThreads + threadIdx.x;
  if (e >= entries) return;
  const int g = group_idx[e];
  if (g < 0 || g >= n_g) return;
  const int64_t row = e / k_g;  // (b, h, i)
  const int64_t bh = row / Nq;
  const int h = static_cast<int>(bh % Hq);
  const int64_t b = bh / Hq;
  const int64_t unit = b * (Hq / r) + h / r;
  __hip_atomic_fetch_or(marks + unit * words + (g >> 5), 1u << (g & 31), __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per (sequence, KV head): ranks of the marked groups.
__global__ __launch_bounds__(kStageThreads) void assign_kernel(const uint32_t* marks, int n_g,
                                                               int words, int cap,
                                                               int32_t* block_table,
                                                               int32_t* page_group,
                                                               int32_t* counts) {
  __shared__ int s_wave[kStageThreads / kWave];
  __shared__ int s_carry;
  const int64_t unit = blockIdx.x;
  const uint32_t* m = marks + unit * words;
  int32_t* table = block_table + unit * n_g;
  int32_t* inv = page_group + unit * cap;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int w0 = 0; w0 < words; w0 += kStageThreads) {
    const int w = w0 + static_cast<int>(threadIdx.x);
    const uint32_t bits = w < words ? m[w] : 0u;
    const int c = __popc(bits);
    // exclusive prefix of c over the workgroup: wave scan, then across waves
    int incl = c;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    int before = s_carry;
    for (int v = 0; v < wave; ++v) before += s_wave[v];
    int rank = before + incl - c;
    if (w < words) {
      for (int j = 0; j < 32; ++j) {
        const int g = w * 32 + j;
        if (g >= n_g) break;
        if ((bits >> j) & 1u) {
          table[g] = static_cast<int32_t>(unit * cap + rank);
          inv[rank] = g;
          ++rank;
        } else {
          table[g] = -1;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x == kStageThreads - 1) s_carry = before + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) counts[unit] = s_carry;
}

// One workgroup per pool page slot of a unit: copy the group's keys and values.
template <typename T>
__global__ __launch_bounds__(kStageThreads) void gather_kernel(const T* K, const T* V, int Hkv,
                                                               int64_t T_len, int D, int G,
                                                               int cap, const int32_t* page_group,
                                                               const int32_t* counts, T* K_pool,
                                                               T* V_pool) {
  const int64_t unit = blockIdx.y;
  const int rank = blockIdx.x;
  if (rank >= counts[unit]) return;
  const int g = page_group[unit * cap + rank];
  const int64_t t0 = static_cast<int64_t>(g) * G;
  const int64_t n_tok = t0 + G <= T_len ? G : T_len - t0;
  const int64_t n16 = n_tok * D * static_cast<int64_t>(sizeof(T)) / 16;  // 16-byte pieces
  const size_t src = (static_cast<size_t>(unit) * T_len + t0) * D;        // unit = b*Hkv + kv
  const size_t dst = (static_cast<size_t>(unit) * cap + rank) * G * D;
  const uint4* ks = reinterpret_cast<const uint4*>(K + src);
  const uint4* vs = reinterpret_cast<const uint4*>(V + src);
  uint4* kd = reinterpret_cast<uint4*>(K_pool + dst);
  uint4* vd = reinterpret_cast<uint4*>(V_pool + dst);
  (void)Hkv;
  // every load of the group in flight before the stores
  constexpr int kPer = 4;
  for (int64_t base = threadIdx.x; base < n16; base += kStageThreads * kPer) {
    uint4 a[kPer], c[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kStageThreads;
      a[u] = c[u] = make_uint4(0, 0, 0, 0);
      if (i < n16) {
        a[u] = ks[i];
        c[u] = vs[i];
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * kStageThreads;
      if (i < n16) {
        kd[i] = a[u];
        vd[i] = c[u];
      }
    }
  }
}

}  // namespace

StagePlan plan_stage(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t T, int G, int k_g) {
  StagePlan s{};
  s.n_g = (T + G - 1) / G;
  s.units = B * Hkv;
  const int64_t rows_per_unit = (Hq / Hkv) * Nq;
  s.cap = rows_per_unit * k_g < s.n_g ? rows_per_unit * k_g : s.n_g;
  s.words = (s.n_g + 31) / 32;
  s.pool_pages = s.units * s.cap;
  return s;
}

hipError_t launch_stage(const StageArgs& a, int dtype, hipStream_t stream) {
  const StagePlan& s = a.plan;
  const int64_t n_marks = s.units * s.words;
  hipLaunchKernelGGL(clear_kernel, dim3(static_cast<unsigned>((n_marks + kStageThreads - 1) /
                                                              kStageThreads)),
                     dim3(kStageThreads), 0, stream, a.marks, n_marks);
  const int64_t entries = a.B * a.Hq * a.Nq * a.k_g;
  hipLaunchKernelGGL(mark_kernel,
                     dim3(static_cast<unsigned>((entries + kStageThreads - 1) / kStageThreads)),
                     dim3(kStageThreads), 0, stream, a.group_idx, entries, a.k_g, a.Hq, a.Nq,
                     a.Hq / a.Hkv, static_cast<int>(s.n_g), static_cast<int>(s.words), a.marks);
  hipLaunchKernelGGL(assign_kernel, dim3(static_cast<unsigned>(s.units)), dim3(kStageThreads), 0,
                     stream, a.marks, static_cast<int>(s.n_g), static_cast<int>(s.words),
                     static_cast<int>(s.cap), a.block_table, a.page_group, a.counts);
  const dim3 grid(static_cast<unsigned>(s.cap), static_cast<unsigned>(s.units));
  if (dtype == kF32) {
    hipLaunchKernelGGL((gather_kernel<float>), grid, dim3(kStageThreads), 0, stream,
                       static_cast<const float*>(a.K), static_cast<const float*>(a.V), a.Hkv, a.T,
                       a.D, a.G, static_cast<int>(s.cap), a.page_group, a.counts,
                       static_cast<float*>(a.K_pool), static_cast<float*>(a.V_pool));
  } else {
    hipLaunchKernelGGL((gather_kernel<uint16_t>), grid, dim3(kStageThreads), 0, stream,
                       static_cast<const uint16_t*>(a.K), static_cast<const uint16_t*>(a.V),
                       a.Hkv, a.T, a.D, a.G, static_cast<int>(s.cap), a.page_group, a.counts,
                       static_cast<uint16_t*>(a.K_pool), static_cast<uint16_t*>(a.V_pool));
  }
  return hipGetLastError();
}

}  // namespace hga

// Device helpers shared by the libhga kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hga {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 / 16-byte lanes
// A lane moves 16 bytes per load: 8 bf16 or 4 f32 elements of one row.
template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kPer16 = 4; };
template <> struct Elem<uint16_t> { static constexpr int kPer16 = 8; };

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Widen one 16-byte chunk to fp32.
__device__ __forceinline__ void widen(const uint4& u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void widen(const uint4& u, float (&x)[4]) {
  x[0] = __uint_as_float(u.x);
  x[1] = __uint_as_float(u.y);
  x[2] = __uint_as_float(u.z);
  x[3] = __uint_as_float(u.w);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------- cross-lane
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N in 1,2,4,8,16,32,64); every lane of a
// group gets the group's total. Within a 16-lane DPP row the butterfly is
// quad xor1, quad xor2, half-row mirror, row mirror.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if constexpr (N >= 16) v += dpp<0x140>(v);  // row_mirror
  if constexpr (N >= 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (N >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Sum/max over lanes that are S, 2S, 4S, ... apart (S a power of two < 64): the
// lanes holding the same column slot of different rows.
template <int S>
__device__ __forceinline__ float across_rows_sum(float v) {
#pragma unroll
  for (int m = S; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
template <int S>
__device__ __forceinline__ float across_rows_max(float v) {
#pragma unroll
  for (int m = S; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int bits_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// ---------------------------------------------------------------- ordering
// Monotone map of a finite float to uint32 (larger float -> larger key); -0 and
// +0 map to the same key. Key 0 never comes out of a finite float, so it marks
// "not a candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0 -> +0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k over the items of one wave. Item e*64 + lane holds key[e] (0 = absent).
// Chooses the k largest keys, equal keys going to the lower item index; returns
// a per-lane bit set (bit e = item e*64+lane chosen). Requires that more than
// k items be present. All lanes of the wave must call it.
template <int E>
__device__ __forceinline__ uint32_t wave_top_k(const uint32_t (&key)[E], int k) {
  // Largest threshold t with #(key >= t) >= k, found bit by bit from the top:
  // that is the k-th largest key. Stop early once exactly k keys are >= t: the
  // chosen set is then fixed whatever the lower bits.
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += __popcll(ballot(key[e] >= t));
    if (cnt >= k) {
      thr = t;
      if (cnt == k) break;
    }
  }
  int above = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) above += __popcll(ballot(key[e] > thr));
  const int need = k - above;  // keys equal to thr still to take, lowest index first
                               // (all of them after an early stop)
  uint32_t chosen = 0;
  int eq_before = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool eq = key[e] == thr;
    const uint64_t eqm = ballot(eq);
    const bool take = key[e] > thr || (eq && eq_before + bits_below(eqm) < need);
    chosen |= static_cast<uint32_t>(take) << e;
    eq_before += __popcll(eqm);
  }
  return chosen;
}

// ---------------------------------------------------------------- grid-level hand-off
// Data one workgroup hands to another goes through agent-scope relaxed atomics:
// on gfx950 those are coherent across the 8 XCDs' L2s by themselves (stores
// write through, loads read the coherent copy), so no workgroup has to write
// back or invalidate its whole L2 as an agent-scope fence would.
__device__ __forceinline__ void store_shared(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every thread of a workgroup after it issued its store_shared()
// results. Returns true in exactly one workgroup of the `total` that share
// `counter`: the last to arrive, which can then read every other workgroup's
// results with load_shared(). That workgroup resets the counter to zero for the
// next call. No workgroup ever waits for another.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned total, bool* s_flag) {
  // Every store of this thread is performed (acknowledged at the coherence
  // point) before the workgroup counts itself in.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == total - 1;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag;
}

}  // namespace hga

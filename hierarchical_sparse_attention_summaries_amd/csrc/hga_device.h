// Device helpers shared by the libhga kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// A raw buffer (stride 0) over `bytes` bytes from p, which must be the same in
// every lane, and 16-byte loads from it at byte offset `off` that read zeros
// past its end (the callers' offsets and sizes are multiples of 16, so a load
// lies wholly inside or wholly outside). Such a load needs no branch around
// it, so the compiler can keep counting it among the loads in flight (a branch
// makes it wait for all). 0x00020000 is the descriptor's fourth word with a
// 32-bit data format, as gfx9-family raw buffer accesses use.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_ld16(__amdgpu_buffer_rsrc_t r, int off) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
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

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, false));
}

// The values of lane l and of lane l ^ 16 (SPAN 16: the other row of a row
// pair) or l ^ 32 (SPAN 32: the other half-wave), as (lower lane's, upper
// lane's), via gfx950's permlane swaps: no LDS round trip.
template <int SPAN>
__device__ __forceinline__ void lane_pair(uint32_t v, uint32_t& lo, uint32_t& hi) {
  static_assert(SPAN == 16 || SPAN == 32, "row-pair or half-wave span");
  if constexpr (SPAN == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    lo = r[0];
    hi = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    lo = r[0];
    hi = r[1];
  }
}
template <int SPAN>
__device__ __forceinline__ float pair_sum(float v) {
  uint32_t lo, hi;
  lane_pair<SPAN>(__float_as_uint(v), lo, hi);
  return __uint_as_float(lo) + __uint_as_float(hi);
}
template <int SPAN>
__device__ __forceinline__ float pair_max(float v) {
  uint32_t lo, hi;
  lane_pair<SPAN>(__float_as_uint(v), lo, hi);
  return fmaxf(__uint_as_float(lo), __uint_as_float(hi));
}

// Sum over aligned groups of N lanes (N in 1,2,4,8,16,32,64); every lane of a
// group gets the group's total. Within a 16-lane DPP row the butterfly runs
// largest span first: row mirror (lane t with 15 - t), half-row mirror (t with
// t ^ 7), quad xor2, quad xor1; then row pairs and half-waves.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 16) v += dpp<0x140>(v);  // row_mirror
  if constexpr (N >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if constexpr (N >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (N >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (N >= 32) v = pair_sum<16>(v);
  if constexpr (N >= 64) v = pair_sum<32>(v);
  return v;
}

// N partial sums per lane over aligned groups of N lanes (N in 2,4,8,16):
// returns, in lane t of a group, the group total of value t % N, with the
// same additions in the same order as group_sum<N> on that value alone (so
// the same bits). Each step keeps the half of its values that its lane's bit
// selects and adds the partner's copy of that half: N - 1 exchanges instead of
// N * log2(N).
template <int N>
__device__ __forceinline__ float group_sum_scatter(const float (&c)[N]) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "2..16 lanes");
  constexpr int H = N / 2;
  const bool hi = (__lane_id() & H) != 0;
  float next[H];
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float keep = hi ? c[k + H] : c[k];
    const float send = hi ? c[k] : c[k + H];
    if constexpr (N == 16) {
      next[k] = keep + dpp<0x140>(send);  // row_mirror: the partner differs in bit 3
    } else if constexpr (N == 8) {
      next[k] = keep + dpp<0x141>(send);  // row_half_mirror: bit 2
    } else if constexpr (N == 4) {
      next[k] = keep + dpp<0x4E>(send);   // quad xor2: bit 1
    } else {
      next[k] = keep + dpp<0xB1>(send);   // quad xor1: bit 0
    }
  }
  if constexpr (H == 1) {
    return next[0];
  } else {
    return group_sum_scatter<H>(next);
  }
}

// Sum/max over lanes that are S, 2S, 4S, ... apart (S a power of two < 64): the
// lanes holding the same column slot of different rows.
template <int S>
__device__ __forceinline__ float across_rows_sum(float v) {
#pragma unroll
  for (int m = S; m < 16; m <<= 1) v += __shfl_xor(v, m, kWave);
  if constexpr (S <= 16) v = pair_sum<16>(v);
  return pair_sum<32>(v);
}
template <int S>
__device__ __forceinline__ float across_rows_max(float v) {
#pragma unroll
  for (int m = S; m < 16; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  if constexpr (S <= 16) v = pair_max<16>(v);
  return pair_max<32>(v);
}

// Whole-wave sum of a 32-bit value; every lane gets the result.
#define HGA_WAVE_REDUCE(NAME, OP)                                   \
  __device__ __forceinline__ uint32_t NAME(uint32_t v) {            \
    v = v OP dpp_u32<0xB1>(v);                                      \
    v = v OP dpp_u32<0x4E>(v);                                      \
    v = v OP dpp_u32<0x141>(v);                                     \
    v = v OP dpp_u32<0x140>(v);                                     \
    uint32_t lo, hi;                                                \
    lane_pair<16>(v, lo, hi);                                       \
    v = lo OP hi;                                                   \
    lane_pair<32>(v, lo, hi);                                       \
    return lo OP hi;                                                \
  }
HGA_WAVE_REDUCE(wave_add, +)
#undef HGA_WAVE_REDUCE

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

// Per-lane bit set over a lane's E selection items (bit e = item e*64 + lane):
// 32 bits while E <= 32, 64 bits above.
template <int E>
using SelMask = typename std::conditional<(E > 32), uint64_t, uint32_t>::type;
static_assert(sizeof(SelMask<64>) * 8 >= 64, "one bit per item");

// Top-k over the items of one wave. Item e*64 + lane holds key[e] (0 = absent).
// Chooses the k largest keys, equal keys going to the lower item index; returns
// a per-lane bit set (bit e = item e*64+lane chosen). Requires that more than
// k items be present. All lanes of the wave must call it.
template <int E>
__device__ __forceinline__ SelMask<E> wave_top_k(const uint32_t (&key)[E], int k) {
  // The k-th largest key is the largest t with #(key >= t) >= k; it is found
  // two bits per step from the top (the three candidate digits are counted
  // independently; the threshold stays in scalar registers). Stop early once
  // exactly k keys are >= t: the chosen set is then fixed whatever the lower
  // bits.
  uint32_t thr = 0;
  for (int bit = 30; bit >= 0; bit -= 2) {
    const uint32_t t1 = thr | (1u << bit), t2 = thr | (2u << bit), t3 = thr | (3u << bit);
    // all compares first, then the counts (a few percent faster than
    // interleaving them)
    uint64_t b1[E], b2[E], b3[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      b3[e] = ballot(key[e] >= t3);
      b2[e] = ballot(key[e] >= t2);
      b1[e] = ballot(key[e] >= t1);
    }
    int c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      c3 += __popcll(b3[e]);
      c2 += __popcll(b2[e]);
      c1 += __popcll(b1[e]);
    }
    int c = -1;
    if (c3 >= k) {
      thr = t3;
      c = c3;
    } else if (c2 >= k) {
      thr = t2;
      c = c2;
    } else if (c1 >= k) {
      thr = t1;
      c = c1;
    }
    thr = __builtin_amdgcn_readfirstlane(thr);
    if (c == k) break;
  }
  int above = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) above += __popcll(ballot(key[e] > thr));
  const int need = k - above;  // keys equal to thr still to take, lowest index first
                               // (all of them after an early stop)
  SelMask<E> chosen = 0;
  int eq_before = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool eq = key[e] == thr;
    const uint64_t eqm = ballot(eq);
    const bool take = key[e] > thr || (eq && eq_before + bits_below(eqm) < need);
    chosen |= static_cast<SelMask<E>>(take) << e;
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
__device__ __forceinline__ void store_shared_i32(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_shared_i32(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A float as a hand-off word in memory that is zero at rest: the bits of x + 0
// (so never -0) with the sign bit flipped, which is never zero, so a reader
// that sees a non-zero word has the value (no flag needed). The round trip
// gives x, or +0 for -0.
__device__ __forceinline__ int32_t handoff_word(float x) {
  return __float_as_int(x + 0.0f) ^ static_cast<int32_t>(0x80000000u);
}
__device__ __forceinline__ float handoff_float(int32_t w) {
  return __int_as_float(w ^ static_cast<int32_t>(0x80000000u));
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

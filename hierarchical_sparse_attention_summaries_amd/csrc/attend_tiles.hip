// Step 3 of HGA (abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709) for many queries per head (chunked prefill): exact attention of
// a tile of query rows over the union of their routed groups, on MFMA.
//
// Neighbouring query rows of one head share many routed groups, so a tile of
// 128 consecutive rows reads each group of the tile's union once (about a
// tenth of what per-row gathers read at a 64K context) and runs the products
// on MFMA 16x16x32 bf16, masking per row: a row takes a group's tokens only if
// it routed the group, and only up to its own position.
//
// Layout, per 16-row block of a wave (a wave has two): S^T = K . Q^T with K
// rows as the A operand and the block's query rows as B, so that each lane
// ends up with 8 scores of one row per group (two 16-token blocks); the online
// softmax keeps (m, l) per row in the 4 lanes that hold it; O^T = V^T . P^T
// with V^T as A and the lane's own probabilities as B (the 32 tokens of a
// group in the lane order the scores came in), so each lane accumulates 32
// dims of its own row and the rescaling stays lane-local. V is staged in LDS
// row-major, as loaded, and its V^T operand comes from gfx950's transposed
// LDS reads. One operand read from LDS serves both row blocks. P enters the
// product rounded to bf16 (each weight within 2^-9 relative; l and the
// accumulation stay fp32).
#include <math.h>

#include "hga_device.h"
#include "hga_internal.h"

namespace hga {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTW = 4;                           // waves per workgroup
constexpr int kRB = 2;                           // 16-row blocks per wave
constexpr int kTR = kTW * kRB * 16;              // query rows per tile (workgroup): 128
constexpr int kTThreads = kTW * kWave;
constexpr int kTG = 32;                          // tokens per group
constexpr int kTD = 128;                         // head dim
constexpr int kSG = 1;                           // groups staged per step
constexpr int kStageTok = kSG * kTG;
constexpr int kKStride = kTD + 8;                // bf16 per staged K row (padded)
// bf16 per staged V row (padded by 32 bytes: the 16 token rows one transposed
// read touches then start 8 banks apart)
constexpr int kVStride = kTD + 16;
constexpr int kTileMaxGroups = 2048;             // groups of the context (mask rows)
constexpr int kNK = kSG * kTG * 16 / kTThreads;  // K (and V) loads per thread per step
static_assert(kNK >= 1, "every thread loads K and V");
static_assert(kTR == 32 * kTW, "one 32-bit mask word per wave");

struct TileLds {
  uint32_t mask[kTileMaxGroups][kTR / 32];       // rows of the tile that routed each group
  int list[kTileMaxGroups];                      // the union, ascending
  alignas(16) uint16_t k[2][kStageTok * kKStride];  // staged K rows, two steps
  alignas(16) uint16_t v[2][kStageTok * kVStride];  // staged V rows, two steps
  int wave_count[kTW];
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Two fp32 values as bf16 (round to nearest even, one conversion instruction).
__device__ __forceinline__ uint32_t bf16_pair(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
}

// gfx950's transposed LDS read of 16-bit data: within each group of 16 lanes,
// lane i receives, in slot j (0..3), element i % 4 of the four at the address
// lane 4j + i / 4 gave (8-byte aligned).
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Workgroup barrier ordering LDS only: unlike __syncthreads(), it does not
// wait for this thread's global loads, so loads issued ahead stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The union's group ids (and, with `bits`, this wave's row bits of each) for
// 64 steps at a time: lane j holds those of step base + j and a step takes
// its own with readlane, so no step waits for an LDS read of its own. Steps
// only ascend.
template <bool kBits>
struct StepWindow {
  int base = -kWave;
  int g = -1;
  uint32_t bits = 0u;
  __device__ __forceinline__ void at(const TileLds& s, int n_u, int wave, int u, int& g_u,
                                     uint32_t& bits_u) {
    if (u - base >= kWave) {  // uniform over the wave
      base = u - u % kWave;
      const int j = base + lane_id();
      g = j < n_u ? s.list[j] : -1;
      if constexpr (kBits) bits = g >= 0 ? s.mask[g][wave] : 0u;
    }
    g_u = __builtin_amdgcn_readlane(g, u - base);
    bits_u = kBits ? __builtin_amdgcn_readlane(bits, u - base) : 0u;
  }
};

// This thread's share of one step (zeros past the union's end or the
// context's end), dims (t % 16) * 8 .. +7 each: K and V of step tokens
// t / 16 + n * (threads / 16).
struct StepRegs {
  uint4 k[kNK], v[kNK];
};

__device__ __forceinline__ void fetch_step(const AttendArgs& a, const TileLds& s, int n_u, int b,
                                           int kv, int wave, int step, StepWindow<false>& win,
                                           StepRegs& r) {
  const int t = static_cast<int>(threadIdx.x);
  const int col = (t % 16) * 8;
  // each of the step's groups as a buffer over the tokens the context holds
  // (a group lies within one page); an empty buffer past the union's end or
  // for a page out of range
  __amdgpu_buffer_rsrc_t rk[kSG], rv[kSG];
#pragma unroll
  for (int gi = 0; gi < kSG; ++gi) {
    const int u = step * kSG + gi;
    int64_t base = -1;
    int n_tok = 0;
    int g_u;
    uint32_t unused;
    win.at(s, n_u, wave, u, g_u, unused);
    if (g_u >= 0) {
      const int t0 = g_u * kTG;
      base = kv_offset(a.kv, b, a.Hkv, kv, a.T, kTD, t0);
      n_tok = min(kTG, a.T - t0);
    }
    const int bytes = base >= 0 ? n_tok * kTD * 2 : 0;
    const int64_t at = base >= 0 ? base : 0;
    rk[gi] = buffer_of(static_cast<const uint16_t*>(a.K) + at, bytes);
    rv[gi] = buffer_of(static_cast<const uint16_t*>(a.V) + at, bytes);
  }
#pragma unroll
  for (int n = 0; n < kNK; ++n) {
    const int tg = t / 16 + n * (kTThreads / 16);  // step token
    const int gi = tg / kTG, x = tg % kTG;
    const int off = (x * kTD + col) * 2;
    r.k[n] = buffer_ld16(rk[gi], off);
    r.v[n] = buffer_ld16(rv[gi], off);
  }
}

__device__ __forceinline__ void stash_step(TileLds& s, int buf, const StepRegs& r) {
  const int t = static_cast<int>(threadIdx.x);
  const int col = (t % 16) * 8;
#pragma unroll
  for (int n = 0; n < kNK; ++n) {
    const int tg = t / 16 + n * (kTThreads / 16);
    *reinterpret_cast<uint4*>(&s.k[buf][tg * kKStride + col]) = r.k[n];
    *reinterpret_cast<uint4*>(&s.v[buf][tg * kVStride + col]) = r.v[n];
  }
}

__global__ __launch_bounds__(kTThreads, 2) void attend_tiles_kernel(AttendArgs a,
                                                                     int tiles_per_head) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.6931471805599453f;
  __shared__ TileLds s;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int tile = static_cast<int>(blockIdx.x) % tiles_per_head;
  const int bh = static_cast<int>(blockIdx.x) / tiles_per_head;  // b * Hq + h
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int kv = h / (a.Hq / a.Hkv);
  const int i0 = tile * kTR;
  const int nrows = min(kTR, a.Nq - i0);
  const int Tb = seq_len_of(a.kv, b, a.T);
  const int n_g = (a.T + kTG - 1) / kTG;
  const size_t row0 = static_cast<size_t>(bh) * a.Nq + i0;  // global row of tile row 0

  // 1. Which rows of the tile routed which group.
  for (int k = tid; k < n_g * (kTR / 32); k += kTThreads) (&s.mask[0][0])[k] = 0u;
  __syncthreads();
  for (int k = tid; k < nrows * a.k_g; k += kTThreads) {
    const int r = k / a.k_g;
    const int g = a.group_idx[(row0 + r) * a.k_g + k % a.k_g];
    if (g >= 0 && g < n_g) atomicOr(&s.mask[g][r >> 5], 1u << (r & 31));
  }
  __syncthreads();

  // 2. The union of the tile's groups, ascending: slot j covers groups
  // [j * threads, +threads), one per thread. A group on a page outside the
  // pool is left out, as if no row had routed it (its keys are not there).
  int n_u = 0;
  for (int base = 0; base < n_g; base += kTThreads) {
    const int g = base + tid;
    bool present = false;
    if (g < n_g) {
#pragma unroll
      for (int w = 0; w < kTR / 32; ++w) present = present || s.mask[g][w] != 0u;
      if (present && a.kv.paged) present = kv_offset(a.kv, b, a.Hkv, kv, a.T, kTD, g * kTG) >= 0;
    }
    const uint64_t m = ballot(present);
    if (lane == 0) s.wave_count[wave] = __popcll(m);
    __syncthreads();
    int before = n_u;
    for (int w = 0; w < wave; ++w) before += s.wave_count[w];
    int total = n_u;
    for (int w = 0; w < kTW; ++w) total += s.wave_count[w];
    if (present) s.list[before + bits_below(m)] = g;
    n_u = total;
    __syncthreads();
  }

  // 3. This lane's query rows (one in each of the wave's 16-row blocks) as B
  // operands; tile row of block rb: wave * 32 + rb * 16 + lane % 16.
  const int a8 = (lane / 16) * 8;          // k offset of this lane's operand slice
  const int a4 = (lane / 16) * 4;          // token / dim offset of its result slice
  bool row_ok[kRB];
  int p_r[kRB];
  uint4 qB[kRB][kTD / 32];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int my_r = wave * 32 + rb * 16 + lane % 16;
    row_ok[rb] = my_r < nrows;
    p_r[rb] = Tb - a.Nq + i0 + my_r;       // its position (rows past the tile: unused)
#pragma unroll
    for (int ks = 0; ks < kTD / 32; ++ks)
      qB[rb][ks] = row_ok[rb] ? ld16(static_cast<const uint16_t*>(a.Q) + (row0 + my_r) * kTD +
                                     ks * 32 + a8)
                              : make_uint4(0, 0, 0, 0);
  }
  const float sl2 = a.scale * kLog2e;

  f32x4 o[kRB][kTD / 16];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int d = 0; d < kTD / 16; ++d) o[rb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[kRB], l[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
  }

  // One step: kSG groups of the union, staged in LDS.
  StepWindow<true> cwin;   // the steps computed
  StepWindow<false> fwin;  // the steps fetched (ahead of those computed)
  auto compute = [&](int step, int buf) {
    int g[kSG];
    uint32_t bits[kSG];  // the wave's 32 rows that routed each group
    uint32_t any = 0u;
#pragma unroll
    for (int gi = 0; gi < kSG; ++gi) {
      cwin.at(s, n_u, wave, step * kSG + gi, g[gi], bits[gi]);
      any |= bits[gi];
    }
    if (any == 0u) return;  // none of the wave's rows takes these groups
    // S^T: 2 blocks of 16 tokens per group x each 16-row block; one K operand
    // read serves both row blocks
    f32x4 sacc[2 * kSG][kRB];
#pragma unroll
    for (int tb = 0; tb < 2 * kSG; ++tb) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sacc[tb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (bits[tb / 2] == 0u) continue;  // uniform over the wave
#pragma unroll
      for (int ks = 0; ks < kTD / 32; ++ks) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const uint4*>(
            &s.k[buf][(tb * 16 + lane % 16) * kKStride + ks * 32 + a8]));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          sacc[tb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, as_bf16x8(qB[rb][ks]),
                                                                 sacc[tb][rb], 0, 0, 0);
      }
    }
    // Per row block: mask (routed group, causal), online softmax. Token x of
    // group g is taken iff the row routed g and x <= p - g * G. The running
    // maximum m is kept in unscaled score units; p = 2^(s * sl2 - m * sl2) with
    // one fused multiply-add.
    float p[kRB][2 * kSG][4];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float mt = -INFINITY;
      float sv[2 * kSG][4];
#pragma unroll
      for (int gi = 0; gi < kSG; ++gi) {
        const bool in = row_ok[rb] && ((bits[gi] >> (rb * 16 + lane % 16)) & 1u);
        const int lim = in ? p_r[rb] - g[gi] * kTG : -1;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tb = 2 * gi + h2;
            sv[tb][i] = (h2 * 16 + a4 + i <= lim) ? sacc[tb][rb][i] : -INFINITY;
            mt = fmaxf(mt, sv[tb][i]);
          }
      }
      mt = pair_max<16>(mt);
      mt = pair_max<32>(mt);
      const float m_new = fmaxf(m[rb], mt);
      // rescale only where a row's running maximum moved (rarely, once warm)
      if (ballot(m_new > m[rb]) != 0u) {
        const float corr =
            m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m[rb] - m_new) * sl2);
        l[rb] *= corr;
#pragma unroll
        for (int d = 0; d < kTD / 16; ++d) o[rb][d] *= corr;
      }
      m[rb] = m_new;
      // rows with nothing yet: p = 0
      const float nm = m_new == -INFINITY ? 0.f : -m_new * sl2;
#pragma unroll
      for (int tb = 0; tb < 2 * kSG; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[rb][tb][i] = __builtin_amdgcn_exp2f(fmaf(sv[tb][i], sl2, nm));
          l[rb] += p[rb][tb][i];
        }
    }
    // O^T += V^T . P^T, one group at a time, P as bf16; one V^T operand read
    // serves both row blocks
#pragma unroll
    for (int gi = 0; gi < kSG; ++gi) {
      if (bits[gi] == 0u) continue;  // uniform over the wave
      bf16x8 ph[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        uint32_t hw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 2 * e;  // operand slots j, j + 1: block 2gi (j < 4) or 2gi + 1
          hw[e] = bf16_pair(p[rb][2 * gi + j / 4][j % 4], p[rb][2 * gi + j / 4][j % 4 + 1]);
        }
        ph[rb] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
      }
#pragma unroll
      for (int d = 0; d < kTD / 16; ++d) {
        // This lane's V^T slice: dim d * 16 + lane % 16, tokens a4 .. a4 + 3 and
        // 16 + a4 .. + 3 of group gi (the token order of its P^T slice). A
        // transposed read hands lane i of each 16-lane group element i % 4 at
        // the address of lane 4j + i / 4 (j = 0..3), so lane j16 of the group
        // points at token a4 + j16 / 4, dims d * 16 + 4 * (j16 % 4) .. + 3.
        const int j16 = lane % 16;
        const uint16_t* src =
            &s.v[buf][(gi * kTG + a4 + j16 / 4) * kVStride + d * 16 + 4 * (j16 % 4)];
        const uint2 x0 = lds_read_tr16(src);
        const uint2 x1 = lds_read_tr16(src + 16 * kVStride);
        const bf16x8 va = as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          o[rb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph[rb], o[rb][d], 0, 0, 0);
      }
    }
  };

  // 4. The union in steps of kSG groups, through two LDS buffers: step st is
  // computed from buffer st % 2 while step st + 1 is stashed into the other,
  // so one barrier per step both publishes st + 1 and frees buffer st % 2;
  // a step's loads go out two computed steps before it is stashed.
  const int n_st = (n_u + kSG - 1) / kSG;
  StepRegs r0, r1;
  fetch_step(a, s, n_u, b, kv, wave, 0, fwin, r0);
  fetch_step(a, s, n_u, b, kv, wave, 1, fwin, r1);
  stash_step(s, 0, r0);
  lds_barrier();
  fetch_step(a, s, n_u, b, kv, wave, 2, fwin, r0);
  for (int st = 0; st < n_st; st += 2) {
    compute(st, 0);
    stash_step(s, 1, r1);
    lds_barrier();
    if (st + 1 >= n_st) break;
    fetch_step(a, s, n_u, b, kv, wave, st + 3, fwin, r1);
    compute(st + 1, 1);
    stash_step(s, 0, r0);
    lds_barrier();
    fetch_step(a, s, n_u, b, kv, wave, st + 4, fwin, r0);
  }

  // 5. Each row's total over its 4 lanes; each lane writes 32 dims of its rows.
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    float lt = pair_sum<16>(l[rb]);
    lt = pair_sum<32>(lt);
    if (row_ok[rb]) {
      const int my_r = wave * 32 + rb * 16 + lane % 16;
      const size_t orow = (row0 + my_r) * kTD;
      uint16_t* O = static_cast<uint16_t*>(a.O);
#pragma unroll
      for (int d = 0; d < kTD / 16; ++d) {
        uint32_t w[2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const float v0 = lt > 0.f ? o[rb][d][2 * z] / lt : 0.f;
          const float v1 = lt > 0.f ? o[rb][d][2 * z + 1] / lt : 0.f;
          w[z] = bf16_bits(v0) | (bf16_bits(v1) << 16);
        }
        *reinterpret_cast<uint2*>(O + orow + d * 16 + a4) = make_uint2(w[0], w[1]);
      }
      if (a.lse && lane < 16)
        a.lse[row0 + my_r] = lt > 0.f ? (m[rb] * sl2 + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

bool use_tile_attend(const AttendArgs& a, int dtype) {
  return dtype == kBF16 && a.D == kTD && a.G == kTG && (a.T + kTG - 1) / kTG <= kTileMaxGroups &&
         a.Nq >= kTR;
}

hipError_t launch_attend_tiles(const AttendArgs& a, hipStream_t stream) {
  const int tiles_per_head = (a.Nq + kTR - 1) / kTR;
  const int64_t grid = static_cast<int64_t>(a.B) * a.Hq * tiles_per_head;
  hipLaunchKernelGGL(attend_tiles_kernel, dim3(static_cast<unsigned>(grid)), dim3(kTThreads), 0,
                     stream, a, tiles_per_head);
  return hipGetLastError();
}

}  // namespace hga

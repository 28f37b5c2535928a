// Step 2 of HGA (abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709) for many queries at once (chunked prefill): scoring every query
// row against the chunk and group summaries is a dense contraction
// Q[rows x D] x S^T[D x (n_chunks + n_groups)] per KV head, run on MFMA; the
// selection then runs one wave per query row.
//
// Precision: Q holds bf16 values (exact as bf16 MFMA operands); each fp32
// summary s is split into bf16 s_hi = rne(s) and s_lo = rne(s - s_hi), and the
// score is q.s_hi + q.s_lo with fp32 accumulation. Products of bf16 values are
// exact in fp32, and s_hi + s_lo carries s to about 2^-17 relative, so the
// scores match an fp32 dot product to ~1e-6 relative: far inside the 1e-3 score
// margin within which routed sets must agree exactly.
//
// Kernel 1 (split): every summary row becomes bf16 (hi, lo) rows once, in the
// MFMA operand layout. Kernel 2 (scores): a workgroup of 4 waves owns 64 query
// rows and walks all columns in 128-column tiles; each wave a 32 x 64 block per
// tile = 2 x 4 MFMA 16x16x32 tiles over D/32 k-steps, two MFMAs (hi, lo) per
// step, the next 16-column block's operands loading meanwhile. Query rows are
// taken head-major (row = head-in-group * Nq + query), so a tile's rows are 64
// consecutive workspace rows; the tile is staged in LDS and written out as
// full contiguous row segments. Kernel 3 (select): one wave per query row,
// the shared selection code.
#include "hga_device.h"
#include "hga_internal.h"
#include "hga_select.h"

#include <stdint.h>

namespace hga {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTileRows = 64;   // per workgroup
constexpr int kTileCols = 128;  // per workgroup

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Round-to-nearest-even fp32 -> bf16 bits, and the rounded value back in fp32.
__device__ __forceinline__ uint32_t rne_bits(float f, float& back) {
  const uint32_t b = bf16_bits(f);
  back = __uint_as_float(b << 16);
  return b;
}

// 8 fp32 -> (hi, lo) bf16x8 with hi + lo ~ x.
__device__ __forceinline__ void split_hi_lo(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float b0, b1, c0, c1;
    const uint32_t h0 = rne_bits(x[2 * i], b0);
    const uint32_t h1 = rne_bits(x[2 * i + 1], b1);
    const uint32_t l0 = rne_bits(x[2 * i] - b0, c0);
    const uint32_t l1 = rne_bits(x[2 * i + 1] - b1, c1);
    h[i] = h0 | (h1 << 16);
    l[i] = l0 | (l1 << 16);
  }
  hi = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
  lo = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
}

// Summary rows (chunks, then groups) of one (sequence, KV head) -> bf16 hi/lo.
template <int D>
__global__ __launch_bounds__(kThreads) void split_kernel(RouteArgs a) {
  const int N = a.n_c + a.n_g;
  const int bkv = blockIdx.y;
  const int idx8 = blockIdx.x * kThreads + threadIdx.x;  // one 8-dim piece per thread
  if (idx8 >= N * (D / 8)) return;
  const int n = idx8 / (D / 8);
  const int d0 = (idx8 % (D / 8)) * 8;
  const float* src = n < a.n_c ? a.chunk_mean + (static_cast<size_t>(bkv) * a.n_c + n) * D
                               : a.group_mean + (static_cast<size_t>(bkv) * a.n_g + n - a.n_c) * D;
  const float4 v0 = *reinterpret_cast<const float4*>(src + d0);
  const float4 v1 = *reinterpret_cast<const float4*>(src + d0 + 4);
  const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  bf16x8 hi, lo;
  split_hi_lo(x, hi, lo);
  uint16_t* base = a.split + static_cast<size_t>(bkv) * 2 * N * D;
  *reinterpret_cast<bf16x8*>(base + static_cast<size_t>(n) * D + d0) = hi;
  *reinterpret_cast<bf16x8*>(base + (static_cast<size_t>(N) + n) * D + d0) = lo;
}

template <int D>
__global__ __launch_bounds__(kThreads) void score_mfma_kernel(RouteArgs a, int n_row_tiles,
                                                              int n_col_tiles) {
  constexpr int KS = D / 32;  // k-steps of the 16x16x32 MFMA
  __shared__ float s_out[kTileRows][kTileCols + 4];  // +4: rows stay 16-byte aligned
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int lr = lane % 16;   // A: row in block; B: column in tile; D: column
  const int lk = lane / 16;   // k sub-block (8 values); D: row quad
  const int rt = blockIdx.x % n_row_tiles;
  const int bkv = blockIdx.x / n_row_tiles;
  const int kv = bkv % a.Hkv;
  const int b = bkv / a.Hkv;
  const int r = a.Hq / a.Hkv;
  const int M = r * a.Nq;               // query rows of this (b, kv head), head-major
  const int N = a.n_c + a.n_g;          // summary rows: chunks, then groups
  const size_t row0 = static_cast<size_t>(b * a.Hq + kv * r) * a.Nq;  // workspace row of rho = 0
  const int wr = (wave / 2) * 32;
  const int wc = (wave % 2) * 64;
  const int row_base = rt * kTileRows + wr;
  const int nrows = min(kTileRows, M - rt * kTileRows);

  // This wave's 32 query rows stay in registers for every column tile.
  uint4 qa[2][KS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int rho = row_base + rb * 16 + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qa[rb][ks] = rho < M ? ld16(static_cast<const uint16_t*>(a.Q) + (row0 + rho) * D + ks * 32 +
                                  lk * 8)
                           : make_uint4(0, 0, 0, 0);
    }
  }
  const uint16_t* hi_base = a.split + static_cast<size_t>(bkv) * 2 * N * D;
  const uint16_t* lo_base = hi_base + static_cast<size_t>(N) * D;

  // B fragments of one 16-column block: KS k-steps of (hi, lo).
  auto load_b = [&](int col, uint4 (&h)[KS], uint4 (&l)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (col < N) {
        h[ks] = ld16(hi_base + static_cast<size_t>(col) * D + ks * 32 + lk * 8);
        l[ks] = ld16(lo_base + static_cast<size_t>(col) * D + ks * 32 + lk * 8);
      } else {
        h[ks] = make_uint4(0, 0, 0, 0);
        l[ks] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  for (int ct = 0; ct < n_col_tiles; ++ct) {
    const int col_base = ct * kTileCols + wc;
    uint4 hA[KS], lA[KS], hB[KS], lB[KS];
    load_b(col_base + lr, hA, lA);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      // next block's fragments in flight while this one runs on MFMA
      if (cb + 1 < 4) load_b(col_base + (cb + 1) * 16 + lr, (cb & 1) ? hA : hB, (cb & 1) ? lA : lB);
      const uint4(&h)[KS] = (cb & 1) ? hB : hA;
      const uint4(&l)[KS] = (cb & 1) ? lB : lA;
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[rb][ks]), as_bf16x8(h[ks]),
                                                            acc[rb], 0, 0, 0);
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[rb][ks]), as_bf16x8(l[ks]),
                                                            acc[rb], 0, 0, 0);
        }
      }
      // D fragment: lane holds rows lk*4 + i of each 16-row block, column lr.
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_out[wr + rb * 16 + lk * 4 + i][wc + cb * 16 + lr] = acc[rb][i] * a.scale;
    }
    __syncthreads();
    // The tile's rows, each a contiguous run of chunk or group columns in its
    // workspace row: one wave per row, four columns per lane, 16-byte stores
    // where the destination allows.
    const int tile_col0 = ct * kTileCols;
    const int ncols = min(kTileCols, N - tile_col0);
    for (int tr = wave; tr < nrows; tr += kThreads / kWave) {
      const size_t wrow = row0 + rt * kTileRows + tr;
      for (int tc = lane * 4; tc < ncols; tc += kWave * 4) {
        const int col = tile_col0 + tc;
        const float4 v = *reinterpret_cast<const float4*>(&s_out[tr][tc]);
        float* dst = col < a.n_c ? a.chunk_scores + wrow * a.n_c + col
                                 : a.group_scores + wrow * a.n_g + (col - a.n_c);
        const bool same_part = (col < a.n_c) == (col + 3 < a.n_c);
        if (tc + 4 <= ncols && same_part && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
          *reinterpret_cast<float4*>(dst) = v;
        } else {
          const float vv[4] = {v.x, v.y, v.z, v.w};
          for (int e = 0; e < 4 && tc + e < ncols; ++e) {
            const int c = col + e;
            if (c < a.n_c) {
              a.chunk_scores[wrow * a.n_c + c] = vv[e];
            } else {
              a.group_scores[wrow * a.n_g + (c - a.n_c)] = vv[e];
            }
          }
        }
      }
    }
    __syncthreads();  // s_out is rewritten by the next tile
  }
}

// ---------------------------------------------------------------------------
// Both levels in one kernel, scores never leaving the chip. A workgroup of
// kFusedThreads / 64 waves owns kFusedRows head-major query rows of one
// (sequence, KV head):
//  1. MFMA scores of the 32 rows against every chunk summary -> LDS;
//  2. each wave selects the chunks of its rows (chunk 0, the row's own chunk L,
//     the k_chunk best between) and marks, per row, each kept chunk's rank;
//  3. MFMA scores against every group summary; a score is kept only if its
//     group lies in a kept chunk of that row (and starts at or before the row's
//     position), and goes straight to the row's candidate slot in LDS (the slot
//     of chunk rank x C/G + group within chunk: candidates in ascending group
//     order, as the selection expects);
//  4. each wave selects the groups of its rows and writes the ids.
// Same scores (same MFMA order) and same selection as the three-kernel path.
constexpr int kFusedRows = 32;
constexpr int kFusedBlocks = kFusedRows / 16;  // 16-row MFMA blocks
constexpr int kFusedThreads = 256;
constexpr int kFusedWaves = kFusedThreads / kWave;

struct FusedLds {
  int stride;  // floats per row of the score area
  size_t scores, kept, rank, bytes;
};
__host__ __device__ inline FusedLds fused_lds(int n_c, int cap, int gpc) {
  FusedLds f{};
  f.stride = n_c > cap * gpc ? n_c : cap * gpc;
  f.scores = 0;
  f.kept = f.scores + static_cast<size_t>(kFusedRows) * f.stride * 4;
  f.rank = f.kept + static_cast<size_t>(kFusedRows) * cap * 4;
  f.bytes = f.rank + static_cast<size_t>(kFusedRows) * ((n_c + 3) / 4 * 4);
  return f;
}

// Workgroups are dealt to the 8 XCDs round-robin by index. Each XCD takes a
// contiguous share of the (sequence, KV head, row tile) list, so that one
// (sequence, KV head)'s split summaries (1.2 MB at 64K, read by every tile of
// it) stay in one or two XCDs' L2 instead of all eight.
__host__ __device__ inline int64_t fused_tiles_per_xcd(int64_t total) { return (total + 7) / 8; }

// Chunk level of one row (wave-wide): the k_c best of chunks 1..L-1 (their
// scores cs[1..L-1], L - 1 > k_c >= 1), ids ascending into kept[1..k_c]. Every
// lane reads a valid score (index clamped), so the reads carry no branch and
// issue together.
template <int EE>
__device__ __forceinline__ void select_chunks(const float* cs, int L, int k_c, int* kept) {
  const int lane = lane_id();
  uint32_t key[EE];
#pragma unroll
  for (int e = 0; e < EE; ++e) {
    const int u = e * kWave + lane;
    const float s = cs[1 + min(u, L - 2)];
    key[e] = u < L - 1 ? order_key(s) : 0u;
  }
  const SelMask<EE> chosen = wave_top_k<EE>(key, k_c);
  int before = 0;
#pragma unroll
  for (int e = 0; e < EE; ++e) {
    const bool ch = (chosen >> e) & 1u;
    const uint64_t m = ballot(ch);
    if (ch) kept[1 + before + bits_below(m)] = 1 + e * kWave + lane;
    before += __popcll(m);
  }
}

template <int D, int E>
__global__ __launch_bounds__(kFusedThreads) void route_prefill_fused_kernel(RouteArgs a,
                                                                            int n_row_tiles,
                                                                            int gpc_shift) {
  constexpr int KS = D / 32;
  constexpr int W = kFusedWaves;
  extern __shared__ float s_lds[];
  const int cap = kept_capacity(a);
  const FusedLds lay = fused_lds(a.n_c, cap, a.gpc);
  float* s_sc = s_lds;
  int* s_kept = reinterpret_cast<int*>(reinterpret_cast<char*>(s_lds) + lay.kept);
  uint8_t* s_rank = reinterpret_cast<uint8_t*>(s_lds) + lay.rank;
  const int rank_stride = (a.n_c + 3) / 4 * 4;
  __shared__ int s_nk[kFusedRows];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int lr = lane % 16;
  const int lk = lane / 16;
  const int64_t total = static_cast<int64_t>(a.B) * a.Hkv * n_row_tiles;
  const int64_t tile = (blockIdx.x % 8) * fused_tiles_per_xcd(total) + blockIdx.x / 8;
  if (tile >= total) return;  // whole workgroup: no barrier follows
  const int rt = static_cast<int>(tile % n_row_tiles);
  const int bkv = static_cast<int>(tile / n_row_tiles);
  const int kv = bkv % a.Hkv;
  const int b = bkv / a.Hkv;
  const int r = a.Hq / a.Hkv;
  const int M = r * a.Nq;
  const int N = a.n_c + a.n_g;
  const size_t row0 = static_cast<size_t>(b * a.Hq + kv * r) * a.Nq;
  const int rho0 = rt * kFusedRows;
  const int nrows = min(kFusedRows, M - rho0);
  const int Tb = route_seq_len(a, b);
  const int gmask = a.gpc - 1;
  auto pos_of = [&](int t) { return Tb - a.Nq + (rho0 + t) % a.Nq; };  // tile row -> p
  auto wrow_of = [&](int t) {  // tile row -> workspace row (b, h, i)
    const int rho = rho0 + t;
    return row0 + static_cast<size_t>(rho / a.Nq) * a.Nq + rho % a.Nq;
  };

  constexpr int RB = kFusedBlocks;
  uint4 qa[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rho = rho0 + rb * 16 + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qa[rb][ks] = rho < M ? ld16(static_cast<const uint16_t*>(a.Q) + (row0 + rho) * D + ks * 32 +
                                  lk * 8)
                           : make_uint4(0, 0, 0, 0);
  }
  const uint16_t* hi_base = a.split + static_cast<size_t>(bkv) * 2 * N * D;
  const uint16_t* lo_base = hi_base + static_cast<size_t>(N) * D;
  // Split rows of column col (zeros at or past `limit`), through buffers over
  // the rows below it, so that no load sits in a branch.
  auto load_b = [&](int col, int limit, uint4 (&h)[KS], uint4 (&l)[KS]) {
    const __amdgpu_buffer_rsrc_t rh = buffer_of(hi_base, limit * D * 2);
    const __amdgpu_buffer_rsrc_t rl = buffer_of(lo_base, limit * D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = (col * D + ks * 32 + lk * 8) * 2;
      h[ks] = buffer_ld16(rh, off);
      l[ks] = buffer_ld16(rl, off);
    }
  };
  auto mfma = [&](const uint4 (&h)[KS], const uint4 (&l)[KS], f32x4 (&acc)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[rb][ks]), as_bf16x8(h[ks]),
                                                          acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[rb][ks]), as_bf16x8(l[ks]),
                                                          acc[rb], 0, 0, 0);
      }
    }
  };
  // 16-column blocks of summary rows [col0, limit): this wave takes blocks
  // wave, wave + W, ...; the next block's operands load while one runs (a
  // block past the end loads zeros without touching memory, so every load is
  // issued unconditionally and the wait before a block's products leaves the
  // next block's loads in flight).
  // consume(first column, acc): lane holds rows rb*16 + lk*4 + i, column + lr.
  auto sweep = [&](int col0, int limit, auto&& consume) {
    const int nblk = (limit - col0 + 15) / 16;
    uint4 hA[KS], lA[KS], hB[KS], lB[KS];
    f32x4 acc[RB];
    int cb = wave;
    load_b(col0 + cb * 16 + lr, limit, hA, lA);
    for (; cb < nblk; cb += 2 * W) {
      load_b(col0 + (cb + W) * 16 + lr, limit, hB, lB);
      __builtin_amdgcn_sched_barrier(0);
      mfma(hA, lA, acc);
      consume(col0 + cb * 16, acc);
      if (cb + W >= nblk) break;
      load_b(col0 + (cb + 2 * W) * 16 + lr, limit, hA, lA);
      __builtin_amdgcn_sched_barrier(0);
      mfma(hB, lB, acc);
      consume(col0 + (cb + W) * 16, acc);
    }
  };

  // 1. chunk scores
  sweep(0, a.n_c, [&](int c0, const f32x4 (&acc)[RB]) {
    const int c = c0 + lr;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = rb * 16 + lk * 4 + i;
        if (t < nrows && c < a.n_c) s_sc[t * lay.stride + c] = acc[rb][i] * a.scale;
      }
  });
  __syncthreads();

  // 2. chunk selection, 8 rows per wave
  for (int t = wave; t < nrows; t += W) {
    const int p = pos_of(t);
    int* kept = s_kept + t * cap;
    uint8_t* rank = s_rank + t * rank_stride;
    for (int c = lane; c < a.n_c; c += kWave) rank[c] = 0xFF;
    int n_kept = 0;
    if (p >= 0) {
      const int L = p / a.C;
      const float* cs = s_sc + t * lay.stride;
      if (L + 1 <= a.k_c + 2) {
        n_kept = L + 1;
        for (int c = lane; c < n_kept; c += kWave) kept[c] = c;
      } else {
        n_kept = a.k_c + 2;
        if (a.k_c > 0) {
          // one key slot fewer when chunks 1..L-1 fit in it (E is sized for
          // the group level)
          bool done = false;
          if constexpr (E > 1) {
            if (L - 1 <= (E - 1) * kWave) {
              select_chunks<E - 1>(cs, L, a.k_c, kept);
              done = true;
            }
          }
          if (!done) select_chunks<E>(cs, L, a.k_c, kept);
        }
        if (lane == 0) {
          kept[0] = 0;
          kept[n_kept - 1] = L;
        }
      }
    }
    wave_lds_sync();
    for (int u = lane; u < n_kept; u += kWave) rank[kept[u]] = static_cast<uint8_t>(u);
    if (a.chunk_idx) {
      int32_t* out = a.chunk_idx + wrow_of(t) * (a.k_c + 2);
      for (int u = lane; u < a.k_c + 2; u += kWave) out[u] = u < n_kept ? kept[u] : -1;
    }
    if (lane == 0) s_nk[t] = n_kept;
  }
  __syncthreads();

  // 3. group scores, straight into each row's candidate slots. A lane's
  // accumulator rows are fixed: their last usable group (-1 for rows past the
  // tile) is worked out once.
  int g_last[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = rb * 16 + lk * 4 + i;
      const int p = t < nrows ? pos_of(t) : -1;
      g_last[rb][i] = p >= 0 ? p / a.G : -1;
    }
  sweep(a.n_c, N, [&](int c0, const f32x4 (&acc)[RB]) {
    const int g = c0 + lr - a.n_c;
    // the chunk's rank in each of the lane's rows, all read at once (the
    // chunk clamped into the table; g <= g_last implies g < n_g)
    const int c = min(g, a.n_g - 1) >> gpc_shift;
    const int slot = g & gmask;
    int rk[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) rk[rb][i] = s_rank[(rb * 16 + lk * 4 + i) * rank_stride + c];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = rb * 16 + lk * 4 + i;
        if (g <= g_last[rb][i] && rk[rb][i] != 0xFF)
          s_sc[t * lay.stride + (rk[rb][i] << gpc_shift) + slot] = acc[rb][i] * a.scale;
      }
  });
  __syncthreads();

  // 4. group selection: candidates after p (or past the end) sit only at the
  // end of a row's list, in its last kept chunk
  for (int t = wave; t < nrows; t += W) {
    const int p = pos_of(t);
    const int n_kept = s_nk[t];
    const int* kept = s_kept + t * cap;
    const int n_cand = n_kept * a.gpc;
    auto gid = [&](int u) { return (kept[u >> gpc_shift] << gpc_shift) + (u & gmask); };
    int n_valid = 0;
    for (int u = lane; u < n_cand; u += kWave) {
      const int g = gid(u);
      n_valid += (g < a.n_g && static_cast<int64_t>(g) * a.G <= p) ? 1 : 0;
    }
    n_valid = static_cast<int>(wave_add(static_cast<uint32_t>(n_valid)));
    const float* gs = s_sc + t * lay.stride;
    uint32_t key[E];
    const int u_last = n_valid > 0 ? n_valid - 1 : 0;  // reads clamped, as above
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int u = e * kWave + lane;
      const float s = gs[min(u, u_last)];
      key[e] = u < n_valid ? order_key(s) : 0u;
    }
    SelMask<E> chosen = 0;
    if (n_valid <= a.k_g) {
#pragma unroll
      for (int e = 0; e < E; ++e) chosen |= static_cast<SelMask<E>>(key[e] != 0u) << e;
    } else {
      chosen = wave_top_k<E>(key, a.k_g);
    }
    int32_t* out = a.group_idx + wrow_of(t) * a.k_g;
    int before = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ch = (chosen >> e) & 1u;
      const uint64_t m = ballot(ch);
      if (ch) out[before + bits_below(m)] = gid(e * kWave + lane);
      before += __popcll(m);
    }
    for (int u = before + lane; u < a.k_g; u += kWave) out[u] = -1;
  }
}

template <int D>
hipError_t launch_fused_d(const RouteArgs& a, int n_row_tiles, int gpc_shift, size_t lds,
                          hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.B) * a.Hkv * n_row_tiles;
  const dim3 grid(static_cast<unsigned>(8 * fused_tiles_per_xcd(total)));
  switch (select_regs(a)) {
#define HGA_FUSED_CASE(EV)                                                                       \
  case EV: {                                                                                     \
    const void* f = reinterpret_cast<const void*>(&route_prefill_fused_kernel<D, EV>);           \
    if (lds > 65536) {                                                                           \
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,    \
                                               static_cast<int>(lds));                           \
      if (e != hipSuccess) return e;                                                             \
    }                                                                                            \
    hipLaunchKernelGGL((route_prefill_fused_kernel<D, EV>), grid, dim3(kFusedThreads), lds,      \
                       stream, a, n_row_tiles, gpc_shift);                                       \
    break;                                                                                       \
  }
    HGA_FUSED_CASE(1)
    HGA_FUSED_CASE(2)
    HGA_FUSED_CASE(3)
    HGA_FUSED_CASE(4)
    HGA_FUSED_CASE(5)
    HGA_FUSED_CASE(6)
    HGA_FUSED_CASE(8)
    HGA_FUSED_CASE(16)
    HGA_FUSED_CASE(32)
    HGA_FUSED_CASE(64)
#undef HGA_FUSED_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;

__global__ __launch_bounds__(kSelThreads) void select_kernel(RouteArgs a, int e_sel, int kept_cap) {
  extern __shared__ int s_kept_all[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int row = blockIdx.x * kSelWaves + wave;
  const int rows = a.B * a.Hq * a.Nq;
  if (row >= rows) return;  // whole wave leaves; no workgroup barrier follows
  const int i = row % a.Nq;
  const int b = row / (a.Hq * a.Nq);
  select_row_e(e_sel, a, row, route_seq_len(a, b) - a.Nq + i, s_kept_all + wave * kept_cap);
}

}  // namespace

bool use_prefill_route(int dtype, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t D) {
  (void)D;
  return dtype == kBF16 && (Hq / Hkv) * Nq >= 64;
}

// The one-kernel form needs a power-of-two C/G (shifts), kept-chunk ranks
// below 255 (one byte each) and its LDS within a workgroup's 160 KiB.
constexpr size_t kMaxWorkgroupLds = 160 * 1024;
bool fused_prefill_ok(const RouteArgs& a) {
  if ((a.gpc & (a.gpc - 1)) != 0) return false;
  const int cap = kept_capacity(a);
  if (cap >= 255) return false;
  return fused_lds(a.n_c, cap, a.gpc).bytes + 256 <= kMaxWorkgroupLds;
}

hipError_t launch_route_prefill(const RouteArgs& a, hipStream_t stream) {
  const int r = a.Hq / a.Hkv;
  const int M = r * a.Nq;
  const int N = a.n_c + a.n_g;
  const dim3 split_grid((N * (a.D / 8) + kThreads - 1) / kThreads, a.B * a.Hkv);
  if (a.D == 64) {
    hipLaunchKernelGGL((split_kernel<64>), split_grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((split_kernel<128>), split_grid, dim3(kThreads), 0, stream, a);
  }
  if (fused_prefill_ok(a)) {
    int shift = 0;
    while ((1 << shift) < a.gpc) ++shift;
    const int n_row_tiles = (M + kFusedRows - 1) / kFusedRows;
    const size_t lds = fused_lds(a.n_c, kept_capacity(a), a.gpc).bytes;
    return a.D == 64 ? launch_fused_d<64>(a, n_row_tiles, shift, lds, stream)
                     : launch_fused_d<128>(a, n_row_tiles, shift, lds, stream);
  }
  const int n_row_tiles = (M + kTileRows - 1) / kTileRows;
  const int n_col_tiles = (N + kTileCols - 1) / kTileCols;
  const int64_t blocks = static_cast<int64_t>(a.B) * a.Hkv * n_row_tiles;
  if (a.D == 64) {
    hipLaunchKernelGGL((score_mfma_kernel<64>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, stream, a, n_row_tiles, n_col_tiles);
  } else {
    hipLaunchKernelGGL((score_mfma_kernel<128>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, stream, a, n_row_tiles, n_col_tiles);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = a.B * a.Hq * a.Nq;
  const int kept_cap = kept_capacity(a);
  const size_t lds = static_cast<size_t>(kSelWaves) * kept_cap * sizeof(int);
  hipLaunchKernelGGL(select_kernel, dim3((rows + kSelWaves - 1) / kSelWaves), dim3(kSelThreads), lds,
                     stream, a, select_regs(a), kept_cap);
  return hipGetLastError();
}

}  // namespace hga

// One-wave selection of one query row's chunks and groups from its scores
// (step 2 of HGA, abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709): the first chunk and the query's own chunk are always kept, plus
// the k_chunk best of the chunks between them; then the k_group best of all
// groups of the kept chunks that start at or before the query. Used by the
// multi-workgroup route (route.hip) and by the select kernel of the
// three-kernel prefill form (route_prefill.hip).
#pragma once

#include "hga_device.h"
#include "hga_internal.h"

namespace hga {

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Selection for one query row, run by one whole wave.
template <int E>
__device__ __forceinline__ void select_row(const RouteArgs& a, int row, int p, int* s_kept) {
  const int lane = lane_id();
  if (p < 0) {  // a query position before the sequence's first key: nothing to route
    if (a.chunk_idx)
      for (int t = lane; t < a.k_c + 2; t += kWave) a.chunk_idx[static_cast<size_t>(row) * (a.k_c + 2) + t] = -1;
    for (int t = lane; t < a.k_g; t += kWave) a.group_idx[static_cast<size_t>(row) * a.k_g + t] = -1;
    return;
  }
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
      // every lane loads a valid score (index clamped; L - 1 > k_c >= 1
      // chunks compete), so the loads carry no branch and are all in flight
      uint32_t key[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int t = e * kWave + lane;
        const float s = load_shared(cs + 1 + min(t, L - 2));
        key[e] = t < L - 1 ? order_key(s) : 0u;
      }
      const SelMask<E> chosen = wave_top_k<E>(key, a.k_c);
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
    const int tc = min(t, n_items - 1);  // every lane loads a valid group's score
    const int g = s_kept[tc / a.gpc] * a.gpc + tc % a.gpc;
    const bool valid = t < n_items && g < a.n_g && static_cast<int64_t>(g) * a.G <= p;
    const float s = load_shared(gs + (g < a.n_g ? g : 0));
    gid[e] = t < n_items ? g : -1;
    key[e] = valid ? order_key(s) : 0u;
    n_valid += __popcll(ballot(valid));
  }
  SelMask<E> chosen = 0;
  if (n_valid <= a.k_g) {
#pragma unroll
    for (int e = 0; e < E; ++e) chosen |= static_cast<SelMask<E>>(key[e] != 0u) << e;
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

__device__ __forceinline__ void select_row_e(int e_sel, const RouteArgs& a, int row, int p,
                                             int* s_kept) {
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

// Keys per lane the selection needs: the smallest compiled variant that holds
// max(middle chunks, candidate groups) items.
inline int select_regs(const RouteArgs& a) {
  const int kept = a.k_c + 2 > a.n_c ? a.n_c : a.k_c + 2;
  const int items = (a.n_c - 2 > kept * a.gpc) ? a.n_c - 2 : kept * a.gpc;
  const int need = (items + kWave - 1) / kWave;
  for (int e : {1, 2, 3, 4, 5, 6, 8, 16, 32}) {
    if (e >= need) return e;
  }
  return 64;
}

// Keys of sequence b (all T unless per-sequence lengths are given).
__device__ __forceinline__ int route_seq_len(const RouteArgs& a, int b) {
  if (!a.seq_lens) return a.T;
  const int t = a.seq_lens[b];
  return t < 0 ? 0 : (t > a.T ? a.T : t);
}

// Chunk ids one query keeps at most (the per-wave LDS list length).
__host__ __device__ inline int kept_capacity(const RouteArgs& a) {
  return a.k_c + 2 > a.n_c ? a.n_c : a.k_c + 2;
}

}  // namespace hga

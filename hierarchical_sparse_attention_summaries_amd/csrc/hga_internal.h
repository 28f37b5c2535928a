// Internal launchers behind the C ABI in include/hga.h. Arguments reaching
// these functions have been validated by the ABI layer (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hga {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// Every workspace starts with kZeroBytes that are zero at rest: every call
// leaves them at zero, so one workspace can serve calls of any shape in turn.
// The first kCounterBytes hold arrival counters (a launch uses at most
// kMaxCounters of them); the rest carries the one-launch decode step's
// hand-off words. Plans put their data after kZeroBytes.
constexpr size_t kCounterBytes = 65536;
constexpr int kMaxCounters = static_cast<int>(kCounterBytes / sizeof(unsigned));
constexpr size_t kZeroBytes = size_t{4} << 20;
// The zero region's last 256 bytes hold the workspace's status word: zero
// while every bounded wait of the one-launch decode step has completed; a
// wait that gave up sets kStatusTimedOut, and the word stays set (every later
// decode step on the workspace then reads no hand-off word and poisons its
// rows) until the caller resets the workspace. Hand-off words end before it.
constexpr size_t kStatusOffset = kZeroBytes - 256;
constexpr int32_t kStatusTimedOut = 1;

// Launch shapes that only tune speed (split counts, grid sizes of kernels
// that never wait for one another) are planned for MI355X/MI350X: 256 CUs in
// 8 XCDs, with no device query, so that size queries work without a device.
constexpr int kPlanCus = 256;

// Largest number of items one wave selects from (middle chunks, or candidate
// groups of the kept chunks), and of chunks one query keeps.
constexpr int kMaxSelectItems = 4096;
constexpr int kMaxKeptChunks = 1024;

// Where the keys/values of token t of (sequence b, KV head kv) live, and how
// many tokens each sequence holds.
struct KvLayout {
  int paged;                   // 0: [B, Hkv, T, D]; 1: pages [n_pages, Hkv, page_tokens, D]
  int page_tokens;             // paged: tokens per page (a multiple of the group size)
  int max_pages;               // paged: columns of block_table
  int n_pages;                 // paged: pages in the pool (ids outside are skipped)
  const int32_t* block_table;  // paged: [B, max_pages] page ids
  const int32_t* seq_lens;     // [B] tokens per sequence (clamped to [0, T]), or null: all T
};

__device__ __forceinline__ int seq_len_of(const KvLayout& L, int b, int T) {
  if (!L.seq_lens) return T;
  const int t = L.seq_lens[b];
  return t < 0 ? 0 : (t > T ? T : t);
}

// Element offset of token t of (b, kv), or -1 if its page id is out of range.
// The G tokens of one group are consecutive rows from there (pages hold whole
// groups).
__device__ __forceinline__ int64_t kv_offset(const KvLayout& L, int b, int Hkv, int kv, int T,
                                             int D, int t) {
  if (!L.paged) return (static_cast<int64_t>(b * Hkv + kv) * T + t) * D;
  const int page = L.block_table[static_cast<int64_t>(b) * L.max_pages + t / L.page_tokens];
  if (page < 0 || page >= L.n_pages) return -1;
  return ((static_cast<int64_t>(page) * Hkv + kv) * L.page_tokens + t % L.page_tokens) * D;
}

// Summaries of chunks [c_first_b, c_first_b + n_chunks) of every (b, kv), where
// c_first_b = max(0, T_b - newest) / C when newest > 0 (the chunks holding each
// sequence's newest `newest` tokens), else c_first_b = c_begin.
hipError_t launch_summaries(const void* K, int dtype, const KvLayout& L, int64_t B, int64_t Hkv,
                            int64_t D, int64_t T, int C, int G, int c_begin, int n_chunks,
                            int64_t newest, float* chunk_mean, float* group_mean,
                            hipStream_t stream);

struct RoutePlan {
  int q_per_block;      // queries of one sequence scored together per KV head
  int n_qblocks;        // ceil(Nq / q_per_block)
  int chunks_per_split; // chunks (and their groups) scored per workgroup
  int n_splits;         // workgroups per (sequence, KV head, query block)
  size_t off_counters, off_chunk_scores, off_group_scores;
  size_t off_split;     // bf16 hi/lo copies of the summaries (prefill path), or 0
  size_t bytes;
};
RoutePlan plan_route(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t T, int C, int G,
                     int k_c, int k_g);

struct RouteArgs {
  const void* Q;
  const float* chunk_mean;
  const float* group_mean;
  int B, Hq, Hkv, Nq, T, D;
  int C, G, gpc, n_c, n_g;
  int k_c, k_g;
  float scale;
  int32_t* chunk_idx;  // may be null
  int32_t* group_idx;
  float* chunk_scores; // workspace [B*Hq*Nq, n_c]
  float* group_scores; // workspace [B*Hq*Nq, n_g]
  unsigned* counters;  // workspace [B*Hkv*n_qblocks]
  uint16_t* split;     // workspace [B*Hkv, 2, n_c + n_g, D] bf16 (hi, lo); prefill path only
  const int32_t* seq_lens;  // [B] or null (all sequences hold T tokens)
  // Decode-step refresh fused into routing: when K is set, the row route first
  // recomputes the summaries of the chunks holding each sequence's newest Nq
  // keys from K (through kv), writes them, and scores with them.
  const void* K;
  KvLayout kv;
};
hipError_t launch_route(const RouteArgs& a, int dtype, const RoutePlan& plan, hipStream_t stream);

// Many query rows per KV head (chunked prefill, bf16): MFMA scoring kernel plus
// a one-wave-per-row select kernel, over the same workspace layout.
bool use_prefill_route(int dtype, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t D);
hipError_t launch_route_prefill(const RouteArgs& a, hipStream_t stream);

// Few query rows (small decode batches): one workgroup per row runs both
// levels on-chip (no workspace use, no cross-workgroup hand-off). Applies to
// at most 1024 rows whose route fits a workgroup's LDS (plus extra_lds bytes
// of other static LDS in the same kernel); `fresh`: the row route also
// refreshes the newest chunks itself (a.K set), which needs Nq <= C and
// C/G <= 16.
bool use_row_route(int64_t B, int64_t Hq, int64_t Nq, int64_t T, int64_t D, int C, int G,
                   int k_c, int k_g, bool fresh, size_t extra_lds = 0);
hipError_t launch_route_rows(const RouteArgs& a, int dtype, hipStream_t stream);

struct AttendPlan {
  int groups_per_wave;
  int n_splits;         // workgroups per query row
  size_t off_counters, off_partials, bytes;
};
// `waves` per workgroup: 4 for the attention launch, 8 inside the fused
// decode-step launch (whose workgroups are sized for routing).
AttendPlan plan_attend(int64_t rows, int64_t D, int G, int k_g, int waves = 4);

struct AttendArgs {
  int32_t* status;     // the workspace's status word (one-launch decode step), or null
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* group_idx;
  void* O;
  float* lse;          // may be null
  int B, Hq, Hkv, Nq, T, D;
  int G, k_g;
  float scale;
  float* partials;     // workspace [rows, n_splits, D + 2]
  unsigned* counters;  // workspace [rows]
  KvLayout kv;
};
hipError_t launch_attend(const AttendArgs& a, int dtype, const AttendPlan& plan,
                         hipStream_t stream);
// Many query rows per head (chunked prefill; bf16, D 128, G 32, at most 2048
// groups): tiles of 128 consecutive rows of one head attend over the union of
// their routed groups on MFMA, each group read once per tile. launch_attend
// takes this path by itself where it applies.
bool use_tile_attend(const AttendArgs& a, int dtype);
hipError_t launch_attend_tiles(const AttendArgs& a, hipStream_t stream);

// Decode step (refresh + score + select + attend) as one launch, every
// workgroup resident at once (at most one per CU): each scores a slice of one
// (sequence, KV head)'s summaries for all its query rows, then selects and
// attends for one (row, split). The scores [rows, n_c + n_g] and the splits'
// partial sums travel as hand-off words in the workspace's zero-at-rest
// region after the counters; no counter is used.
// Attention plan inside the one-launch decode step (8 waves per workgroup) on
// a device of `cus` compute units.
AttendPlan plan_decode_attend(int64_t rows, int64_t D, int k_g, int cus);
// Whether the one-launch form applies on a device of `cus` compute units: the
// grid fits one workgroup per CU, the refresh touches at most two chunks of
// at most 16 groups, the step's hand-off words fit the zero-at-rest region,
// and the row's scores and selection fit the LDS.
bool decode_step_one_launch(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t T, int64_t D,
                            int C, int G, int k_c, int k_g, int cus);
// Workspace bytes of the one-launch form.
size_t decode_step_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t D, int k_g);
hipError_t launch_decode_step(const RouteArgs& ra, const AttendArgs& aa, const AttendPlan& plan,
                              int dtype, void* workspace, int cus, hipStream_t stream);

// Host-memory tier: the routed groups of each (sequence, KV head), over all
// its query rows, copied once into a device pool of [pool_pages, G, D] pages;
// unit = sequence * Hkv + KV head owns pool pages [unit * cap, unit * cap +
// count[unit]) in ascending group order.
struct StagePlan {
  int64_t n_g, units, cap, words, pool_pages;
};
StagePlan plan_stage(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t T, int G, int k_g);
struct StageArgs {
  const void* K;
  const void* V;
  void* K_pool;
  void* V_pool;
  const int32_t* group_idx;
  int64_t B;
  int Hq, Hkv, Nq;
  int64_t T;
  int D, G, k_g;
  uint32_t* marks;       // workspace [units, words]
  int32_t* block_table;  // workspace [units, n_g]: pool page of each group, or -1
  int32_t* page_group;   // workspace [units, cap]: group of each page
  int32_t* counts;       // workspace [units]: pages used
  StagePlan plan;
};
hipError_t launch_stage(const StageArgs& a, int dtype, hipStream_t stream);

// Compute units of the current device (queried once per device), or -1 if
// there is no device or it cannot be queried.
int device_cu_count();
// Compute units every workgroup of one launch may count on holding at once:
// the device's, or 0 when a CU mask in the environment (HSA_CU_MASK,
// ROC_GLOBAL_CU_MASK) may hide some of them from this process's queues.
int resident_cu_count();

}  // namespace hga

#include "hga.h"

namespace hga {

// hga_decode_step_ex with an optional clear of the workspace's zero region
// (enqueued first, once every argument has been checked).
int decode_step_call(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                     const void* K, const void* V, int32_t dtype, float* chunk_mean,
                     float* group_mean, int32_t chunk, int32_t group, int32_t k_chunk,
                     int32_t k_group, float scale, int32_t* chunk_idx, int32_t* group_idx,
                     void* O, float* lse, void* workspace, size_t workspace_bytes,
                     bool clear_first, void* stream);

// Zero-fills `bytes` bytes (a multiple of 16, 16-byte aligned) with a kernel
// (no memset node, so it can be captured in a graph).
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

}  // namespace hga

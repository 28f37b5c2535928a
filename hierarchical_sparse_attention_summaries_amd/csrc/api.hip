// C ABI of libhga (declared in include/hga.h): argument checks on the host,
// then stream-ordered launches. Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <initializer_list>

#include "hga.h"
#include "hga_internal.h"

namespace hga {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0: not queried yet
}  // namespace

int device_cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int known = g_cus[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1)
    return -1;
  if (dev < kMaxDevices) g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

int resident_cu_count() {
  // A CU mask restricts the CUs a process's queues may use, and the device
  // attribute does not show it: then no launch may count on co-residency.
  static const bool masked = std::getenv("HSA_CU_MASK") != nullptr ||
                             std::getenv("ROC_GLOBAL_CU_MASK") != nullptr;
  if (masked) return 0;
  const int n = device_cu_count();
  return n > 0 ? n : 0;
}

namespace {
__global__ void zero_fill_kernel(uint4* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}
}  // namespace

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 16;
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 1024));
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<uint4*>(p), n);
  return hipGetLastError();
}

}  // namespace hga

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the product of non-negative factors is below `limit`, without
// overflowing on the way (any factor may be as large as the caller passes).
bool product_below(std::initializer_list<int64_t> factors, int64_t limit) {
  int64_t p = 1;
  for (const int64_t f : factors)
    if (f < 0 || __builtin_mul_overflow(p, f, &p)) return false;
  return p < limit;
}

int dtype_ok(int32_t dtype) { return dtype == HGA_F32 || dtype == HGA_BF16; }

int check_chunking(int64_t T, int32_t chunk, int32_t group) {
  if (chunk < 1 || group < 1 || chunk % group != 0) return HGA_ERR_PARAM;
  if (group > 65536 || chunk / group > 512) return HGA_ERR_PARAM;
  if (T < 1 || T >= kMaxDim) return HGA_ERR_SHAPE;
  return HGA_OK;
}

int check_shape(const hga_shape* s) {
  if (!s) return HGA_ERR_NULL;
  if (s->batch < 1 || s->q_heads < 1 || s->kv_heads < 1 || s->n_queries < 1 || s->seq_len < 1)
    return HGA_ERR_SHAPE;
  if (s->q_heads % s->kv_heads != 0) return HGA_ERR_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return HGA_ERR_SHAPE;
  if (s->n_queries > s->seq_len) return HGA_ERR_SHAPE;
  if (s->batch >= kMaxDim || s->q_heads >= kMaxDim || s->seq_len >= kMaxDim ||
      !product_below({s->batch, s->q_heads, s->n_queries}, kMaxDim) ||
      !product_below({s->batch, s->kv_heads, s->seq_len}, int64_t(1) << 40))
    return HGA_ERR_SHAPE;
  return HGA_OK;
}

int check_route_params(const hga_shape* s, int32_t chunk, int32_t group, int32_t k_chunk,
                       int32_t k_group) {
  int st = check_chunking(s->seq_len, chunk, group);
  if (st != HGA_OK) return st;
  if (k_chunk < 0 || k_group < 1) return HGA_ERR_PARAM;
  const int64_t n_c = (s->seq_len + chunk - 1) / chunk;
  const int64_t gpc = chunk / group;
  const int64_t n_g = (s->seq_len + group - 1) / group;
  const int64_t kept = std::min<int64_t>(int64_t(k_chunk) + 2, n_c);
  if (n_c - 2 > hga::kMaxSelectItems || kept * gpc > hga::kMaxSelectItems ||
      kept > hga::kMaxKeptChunks)
    return HGA_ERR_UNSUPPORTED;
  if (!product_below({s->batch, s->q_heads, s->n_queries, n_c + n_g}, int64_t(1) << 40))
    return HGA_ERR_SHAPE;
  return HGA_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

float default_scale(float scale, int64_t D) {
  return scale > 0.f ? scale : 1.0f / sqrtf(static_cast<float>(D));
}

hga::RouteArgs route_args(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                          const float* chunk_mean, const float* group_mean, int32_t chunk,
                          int32_t group, int32_t k_chunk, int32_t k_group, float scale,
                          int32_t* chunk_idx, int32_t* group_idx, void* workspace,
                          const hga::RoutePlan& plan) {
  hga::RouteArgs a{};
  a.Q = Q;
  a.chunk_mean = chunk_mean;
  a.group_mean = group_mean;
  a.B = static_cast<int>(shape->batch);
  a.Hq = static_cast<int>(shape->q_heads);
  a.Hkv = static_cast<int>(shape->kv_heads);
  a.Nq = static_cast<int>(shape->n_queries);
  a.T = static_cast<int>(shape->seq_len);
  a.D = static_cast<int>(shape->head_dim);
  a.C = chunk;
  a.G = group;
  a.gpc = chunk / group;
  a.n_c = static_cast<int>((shape->seq_len + chunk - 1) / chunk);
  a.n_g = static_cast<int>((shape->seq_len + group - 1) / group);
  a.k_c = k_chunk;
  a.k_g = k_group;
  a.scale = default_scale(scale, shape->head_dim);
  a.chunk_idx = chunk_idx;
  a.group_idx = group_idx;
  char* ws = static_cast<char*>(workspace);
  a.counters = reinterpret_cast<unsigned*>(ws + plan.off_counters);
  a.chunk_scores = reinterpret_cast<float*>(ws + plan.off_chunk_scores);
  a.group_scores = reinterpret_cast<float*>(ws + plan.off_group_scores);
  a.split = plan.off_split ? reinterpret_cast<uint16_t*>(ws + plan.off_split) : nullptr;
  a.seq_lens = layout ? layout->seq_lens : nullptr;
  return a;
}

hga::AttendArgs attend_args(const hga_shape* shape, const hga::KvLayout& L, const void* Q,
                            const void* K, const void* V, const int32_t* group_idx,
                            int32_t k_group, int32_t group, float scale, void* O, float* lse,
                            void* workspace, const hga::AttendPlan& plan) {
  hga::AttendArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.group_idx = group_idx;
  a.O = O;
  a.lse = lse;
  a.B = static_cast<int>(shape->batch);
  a.Hq = static_cast<int>(shape->q_heads);
  a.Hkv = static_cast<int>(shape->kv_heads);
  a.Nq = static_cast<int>(shape->n_queries);
  a.T = static_cast<int>(shape->seq_len);
  a.D = static_cast<int>(shape->head_dim);
  a.G = group;
  a.k_g = k_group;
  a.scale = default_scale(scale, shape->head_dim);
  char* ws = static_cast<char*>(workspace);
  a.counters = reinterpret_cast<unsigned*>(ws + plan.off_counters);
  a.partials = reinterpret_cast<float*>(ws + plan.off_partials);
  a.kv = L;
  return a;
}

// Whether hga_route_fresh_ex refreshes inside the row route (one launch).
bool row_fresh_fused(const hga_shape* s, int32_t dtype, int32_t chunk, int32_t group,
                     int32_t k_chunk, int32_t k_group) {
  return hga::use_row_route(s->batch, s->q_heads, s->n_queries, s->seq_len, s->head_dim, chunk,
                            group, k_chunk, k_group, true) &&
         !(dtype == HGA_BF16 &&
           hga::use_prefill_route(dtype, s->q_heads, s->kv_heads, s->n_queries, s->head_dim));
}

// Whether hga_decode_step_ex runs as one launch (small batches) on a device
// whose workgroups can all hold `cus` compute units at once.
bool decode_one_launch(const hga_shape* s, int32_t chunk, int32_t group, int32_t k_chunk,
                       int32_t k_group, int cus) {
  return hga::decode_step_one_launch(s->batch, s->q_heads, s->kv_heads, s->n_queries, s->seq_len,
                                     s->head_dim, chunk, group, k_chunk, k_group, cus);
}

// Workspace of hga_decode_step_ex: the larger of the two-call form (routing,
// then attention in stream order over the same workspace) and the one-launch
// form (its score and partial words sit in the zero-at-rest region every
// workspace begins with).
size_t decode_workspace_bytes(const hga_shape* s, int32_t chunk, int32_t group, int32_t k_chunk,
                              int32_t k_group) {
  const int64_t rows = s->batch * s->q_heads * s->n_queries;
  return std::max({hga::plan_route(s->batch, s->q_heads, s->kv_heads, s->n_queries, s->seq_len,
                                   chunk, group, k_chunk, k_group)
                       .bytes,
                   hga::plan_attend(rows, s->head_dim, group, k_group).bytes,
                   hga::decode_step_bytes(s->batch, s->q_heads, s->n_queries, s->head_dim,
                                          k_group)});
}

// Checks a caller's K/V layout against the capacity T and group size and
// converts it; NULL means dense with every sequence holding T keys.
int to_layout(const hga_kv_layout* in, int64_t T, int32_t group, hga::KvLayout* out) {
  *out = hga::KvLayout{};
  if (!in) return HGA_OK;
  out->seq_lens = in->seq_lens;
  if (in->kind == HGA_KV_DENSE) return HGA_OK;
  if (in->kind != HGA_KV_PAGED) return HGA_ERR_PARAM;
  if (!in->block_table) return HGA_ERR_NULL;
  if (in->page_tokens < 1 || group < 1 || in->page_tokens % group != 0 || in->n_pages < 1 ||
      in->max_pages < 1)
    return HGA_ERR_PARAM;
  if (static_cast<int64_t>(in->max_pages) * in->page_tokens < T) return HGA_ERR_PARAM;
  out->paged = 1;
  out->page_tokens = in->page_tokens;
  out->max_pages = in->max_pages;
  out->n_pages = in->n_pages;
  out->block_table = in->block_table;
  return HGA_OK;
}

}  // namespace

extern "C" {

int hga_abi_version(void) { return HGA_ABI_VERSION; }

size_t hga_workspace_zero_bytes(void) { return hga::kZeroBytes; }

const char* hga_status_str(int status) {
  switch (status) {
    case HGA_OK: return "ok";
    case HGA_ERR_NULL: return "a required pointer is NULL";
    case HGA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case HGA_ERR_DTYPE: return "unknown dtype";
    case HGA_ERR_LAYOUT: return "a pointer is not 16-byte aligned";
    case HGA_ERR_PARAM: return "chunk/group/k_chunk/k_group/range out of range";
    case HGA_ERR_WORKSPACE: return "workspace too small";
    case HGA_ERR_HIP: return "HIP call or kernel launch failed";
    case HGA_ERR_UNSUPPORTED: return "request not supported by this build";
    case HGA_ERR_TIMEOUT:
      return "a bounded wait inside a decode step gave up; its rows are NaN; reset the workspace";
    default: return "unknown status";
  }
}

int hga_summary_counts(int64_t seq_len, int32_t chunk, int32_t group, int64_t* n_chunks,
                       int64_t* n_groups) {
  const int st = check_chunking(seq_len, chunk, group);
  if (st != HGA_OK) return st;
  if (n_chunks) *n_chunks = (seq_len + chunk - 1) / chunk;
  if (n_groups) *n_groups = (seq_len + group - 1) / group;
  return HGA_OK;
}

static int summaries_common(const void* K, int32_t dtype, const hga_kv_layout* layout,
                            int64_t batch, int64_t kv_heads, int64_t seq_len, int64_t head_dim,
                            int32_t chunk, int32_t group, int64_t t_begin, int64_t t_end,
                            int64_t newest, float* chunk_mean, float* group_mean, void* stream) {
  if (!K || !chunk_mean || !group_mean) return HGA_ERR_NULL;
  if (!dtype_ok(dtype)) return HGA_ERR_DTYPE;
  if (batch < 1 || kv_heads < 1 || batch >= kMaxDim || kv_heads >= kMaxDim) return HGA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return HGA_ERR_SHAPE;
  int st = check_chunking(seq_len, chunk, group);
  if (st != HGA_OK) return st;
  if (!product_below({batch, kv_heads, seq_len}, int64_t(1) << 40)) return HGA_ERR_SHAPE;
  hga::KvLayout L;
  st = to_layout(layout, seq_len, group, &L);
  if (st != HGA_OK) return st;
  if (!aligned16(K) || !aligned16(chunk_mean) || !aligned16(group_mean)) return HGA_ERR_LAYOUT;
  const int64_t n_c = (seq_len + chunk - 1) / chunk;
  int64_t c_begin = 0, n_chunks = n_c;
  if (newest > 0) {
    if (newest > seq_len) return HGA_ERR_PARAM;
    n_chunks = std::min<int64_t>(n_c, (newest + chunk - 1) / chunk + 1);
  } else {
    if (t_begin < 0 || t_end > seq_len || t_begin >= t_end) return HGA_ERR_PARAM;
    c_begin = t_begin / chunk;
    n_chunks = (t_end + chunk - 1) / chunk - c_begin;
  }
  if (!product_below({batch, kv_heads, n_chunks}, kMaxDim)) return HGA_ERR_SHAPE;
  const hipError_t e = hga::launch_summaries(K, dtype, L, batch, kv_heads, head_dim, seq_len,
                                             chunk, group, static_cast<int>(c_begin),
                                             static_cast<int>(n_chunks), newest, chunk_mean,
                                             group_mean, as_stream(stream));
  return e == hipSuccess ? HGA_OK : HGA_ERR_HIP;
}

int hga_build_summaries(const void* K, int32_t dtype, int64_t batch, int64_t kv_heads,
                        int64_t seq_len, int64_t head_dim, int32_t chunk, int32_t group,
                        float* chunk_mean, float* group_mean, void* stream) {
  return summaries_common(K, dtype, nullptr, batch, kv_heads, seq_len, head_dim, chunk, group, 0,
                          seq_len, 0, chunk_mean, group_mean, stream);
}

int hga_update_summaries(const void* K, int32_t dtype, int64_t batch, int64_t kv_heads,
                         int64_t seq_len, int64_t head_dim, int32_t chunk, int32_t group,
                         int64_t t_begin, int64_t t_end, float* chunk_mean, float* group_mean,
                         void* stream) {
  return summaries_common(K, dtype, nullptr, batch, kv_heads, seq_len, head_dim, chunk, group,
                          t_begin, t_end, 0, chunk_mean, group_mean, stream);
}

int hga_build_summaries_ex(const void* K, int32_t dtype, const hga_kv_layout* layout,
                           int64_t batch, int64_t kv_heads, int64_t seq_len, int64_t head_dim,
                           int32_t chunk, int32_t group, float* chunk_mean, float* group_mean,
                           void* stream) {
  return summaries_common(K, dtype, layout, batch, kv_heads, seq_len, head_dim, chunk, group, 0,
                          seq_len, 0, chunk_mean, group_mean, stream);
}

int hga_update_summaries_ex(const void* K, int32_t dtype, const hga_kv_layout* layout,
                            int64_t batch, int64_t kv_heads, int64_t seq_len, int64_t head_dim,
                            int32_t chunk, int32_t group, int64_t newest, float* chunk_mean,
                            float* group_mean, void* stream) {
  if (newest < 1) return HGA_ERR_PARAM;
  return summaries_common(K, dtype, layout, batch, kv_heads, seq_len, head_dim, chunk, group, 0,
                          0, newest, chunk_mean, group_mean, stream);
}

int hga_route_workspace_size(const hga_shape* shape, int32_t chunk, int32_t group,
                             int32_t k_chunk, int32_t k_group, size_t* bytes) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!bytes) return HGA_ERR_NULL;
  st = check_route_params(shape, chunk, group, k_chunk, k_group);
  if (st != HGA_OK) return st;
  *bytes = hga::plan_route(shape->batch, shape->q_heads, shape->kv_heads, shape->n_queries,
                           shape->seq_len, chunk, group, k_chunk, k_group)
               .bytes;
  return HGA_OK;
}

int hga_route(const hga_shape* shape, const void* Q, int32_t dtype, const float* chunk_mean,
              const float* group_mean, int32_t chunk, int32_t group, int32_t k_chunk,
              int32_t k_group, float scale, int32_t* chunk_idx, int32_t* group_idx,
              void* workspace, size_t workspace_bytes, void* stream) {
  return hga_route_ex(shape, nullptr, Q, dtype, chunk_mean, group_mean, chunk, group, k_chunk,
                      k_group, scale, chunk_idx, group_idx, workspace, workspace_bytes, stream);
}

// Routing; with K_fresh, the row route also refreshes each sequence's newest
// Nq keys' chunks from K_fresh (laid out as kv_fresh) before scoring.
static int route_impl(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                      int32_t dtype, const float* chunk_mean, const float* group_mean,
                      int32_t chunk, int32_t group, int32_t k_chunk, int32_t k_group, float scale,
                      int32_t* chunk_idx, int32_t* group_idx, void* workspace,
                      size_t workspace_bytes, void* stream, const void* K_fresh,
                      const hga::KvLayout* kv_fresh);

int hga_route_ex(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                 int32_t dtype, const float* chunk_mean, const float* group_mean, int32_t chunk,
                 int32_t group, int32_t k_chunk, int32_t k_group, float scale,
                 int32_t* chunk_idx, int32_t* group_idx, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return route_impl(shape, layout, Q, dtype, chunk_mean, group_mean, chunk, group, k_chunk,
                    k_group, scale, chunk_idx, group_idx, workspace, workspace_bytes, stream,
                    nullptr, nullptr);
}

int hga_route_fresh_ex(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                       const void* K, int32_t dtype, float* chunk_mean, float* group_mean,
                       int32_t chunk, int32_t group, int32_t k_chunk, int32_t k_group,
                       float scale, int32_t* chunk_idx, int32_t* group_idx, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!K) return HGA_ERR_NULL;
  if (!aligned16(K)) return HGA_ERR_LAYOUT;
  st = check_route_params(shape, chunk, group, k_chunk, k_group);
  if (st != HGA_OK) return st;
  hga::KvLayout L;
  st = to_layout(layout, shape->seq_len, group, &L);
  if (st != HGA_OK) return st;
  if (!row_fresh_fused(shape, dtype, chunk, group, k_chunk, k_group)) {
    // two launches: refresh, then route
    st = summaries_common(K, dtype, layout, shape->batch, shape->kv_heads, shape->seq_len,
                          shape->head_dim, chunk, group, 0, 0, shape->n_queries, chunk_mean,
                          group_mean, stream);
    if (st != HGA_OK) return st;
    return route_impl(shape, layout, Q, dtype, chunk_mean, group_mean, chunk, group, k_chunk,
                      k_group, scale, chunk_idx, group_idx, workspace, workspace_bytes, stream,
                      nullptr, nullptr);
  }
  return route_impl(shape, layout, Q, dtype, chunk_mean, group_mean, chunk, group, k_chunk,
                    k_group, scale, chunk_idx, group_idx, workspace, workspace_bytes, stream, K,
                    &L);
}

static int route_impl(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                      int32_t dtype, const float* chunk_mean, const float* group_mean,
                      int32_t chunk, int32_t group, int32_t k_chunk, int32_t k_group, float scale,
                      int32_t* chunk_idx, int32_t* group_idx, void* workspace,
                      size_t workspace_bytes, void* stream, const void* K_fresh,
                      const hga::KvLayout* kv_fresh) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (layout && layout->kind != HGA_KV_DENSE && layout->kind != HGA_KV_PAGED) return HGA_ERR_PARAM;
  if (!Q || !chunk_mean || !group_mean || !group_idx || !workspace) return HGA_ERR_NULL;
  if (!dtype_ok(dtype)) return HGA_ERR_DTYPE;
  st = check_route_params(shape, chunk, group, k_chunk, k_group);
  if (st != HGA_OK) return st;
  if (!aligned16(Q) || !aligned16(chunk_mean) || !aligned16(group_mean) || !aligned16(workspace))
    return HGA_ERR_LAYOUT;
  const hga::RoutePlan plan = hga::plan_route(shape->batch, shape->q_heads, shape->kv_heads,
                                              shape->n_queries, shape->seq_len, chunk, group,
                                              k_chunk, k_group);
  if (workspace_bytes < plan.bytes) return HGA_ERR_WORKSPACE;
  hga::RouteArgs a = route_args(shape, layout, Q, chunk_mean, group_mean, chunk, group, k_chunk,
                                k_group, scale, chunk_idx, group_idx, workspace, plan);
  a.K = K_fresh;
  if (kv_fresh) a.kv = *kv_fresh;
  hipError_t e;
  if (a.split && hga::use_prefill_route(dtype, shape->q_heads, shape->kv_heads,
                                        shape->n_queries, shape->head_dim)) {
    e = hga::launch_route_prefill(a, as_stream(stream));
  } else if (a.K || hga::use_row_route(shape->batch, shape->q_heads, shape->n_queries,
                                       shape->seq_len, shape->head_dim, chunk, group, k_chunk,
                                       k_group, false)) {
    e = hga::launch_route_rows(a, dtype, as_stream(stream));
  } else {
    e = hga::launch_route(a, dtype, plan, as_stream(stream));
  }
  return e == hipSuccess ? HGA_OK : HGA_ERR_HIP;
}

int hga_attend_workspace_size(const hga_shape* shape, int32_t group, int32_t k_group,
                              size_t* bytes) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!bytes) return HGA_ERR_NULL;
  if (group < 1 || group > 65536 || k_group < 1) return HGA_ERR_PARAM;
  const int64_t rows = shape->batch * shape->q_heads * shape->n_queries;
  *bytes = hga::plan_attend(rows, shape->head_dim, group, k_group).bytes;
  return HGA_OK;
}

int hga_attend(const hga_shape* shape, const void* Q, const void* K, const void* V,
               int32_t dtype, const int32_t* group_idx, int32_t k_group, int32_t group,
               float scale, void* O, float* lse, void* workspace, size_t workspace_bytes,
               void* stream) {
  return hga_attend_ex(shape, nullptr, Q, K, V, dtype, group_idx, k_group, group, scale, O, lse,
                       workspace, workspace_bytes, stream);
}

int hga_attend_ex(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                  const void* K, const void* V, int32_t dtype, const int32_t* group_idx,
                  int32_t k_group, int32_t group, float scale, void* O, float* lse,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !K || !V || !group_idx || !O || !workspace) return HGA_ERR_NULL;
  if (!dtype_ok(dtype)) return HGA_ERR_DTYPE;
  if (group < 1 || group > 65536 || k_group < 1) return HGA_ERR_PARAM;
  hga::KvLayout L;
  st = to_layout(layout, shape->seq_len, group, &L);
  if (st != HGA_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(workspace))
    return HGA_ERR_LAYOUT;
  const int64_t rows = shape->batch * shape->q_heads * shape->n_queries;
  const hga::AttendPlan plan = hga::plan_attend(rows, shape->head_dim, group, k_group);
  if (workspace_bytes < plan.bytes) return HGA_ERR_WORKSPACE;
  if (rows * plan.n_splits >= kMaxDim) return HGA_ERR_SHAPE;
  const hga::AttendArgs a = attend_args(shape, L, Q, K, V, group_idx, k_group, group, scale, O,
                                        lse, workspace, plan);
  const hipError_t e = hga::launch_attend(a, dtype, plan, as_stream(stream));
  return e == hipSuccess ? HGA_OK : HGA_ERR_HIP;
}

int hga_decode_step_workspace_size(const hga_shape* shape, int32_t chunk, int32_t group,
                                   int32_t k_chunk, int32_t k_group, size_t* bytes) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!bytes) return HGA_ERR_NULL;
  st = check_route_params(shape, chunk, group, k_chunk, k_group);
  if (st != HGA_OK) return st;
  *bytes = decode_workspace_bytes(shape, chunk, group, k_chunk, k_group);
  return HGA_OK;
}

// Workspace of hga_attend_staged: the attention's (counters first), then the
// staging tables.
struct StagedWorkspace {
  hga::StagePlan stage;
  hga::AttendPlan attend;
  size_t marks, table, pages, counts, bytes;
};
StagedWorkspace staged_workspace(const hga_shape* s, int32_t group, int32_t k_group) {
  StagedWorkspace w{};
  w.stage = hga::plan_stage(s->batch, s->q_heads, s->kv_heads, s->n_queries, s->seq_len, group,
                            k_group);
  const int64_t rows = s->batch * s->q_heads * s->n_queries;
  w.attend = hga::plan_attend(rows, s->head_dim, group, k_group);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  w.marks = up(w.attend.bytes);
  w.table = up(w.marks + static_cast<size_t>(w.stage.units * w.stage.words) * 4);
  w.pages = up(w.table + static_cast<size_t>(w.stage.units * w.stage.n_g) * 4);
  w.counts = up(w.pages + static_cast<size_t>(w.stage.units * w.stage.cap) * 4);
  w.bytes = up(w.counts + static_cast<size_t>(w.stage.units) * 4);
  return w;
}

int hga_attend_staged_sizes(const hga_shape* shape, int32_t group, int32_t k_group,
                            int64_t* pool_pages, size_t* workspace_bytes) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!pool_pages || !workspace_bytes) return HGA_ERR_NULL;
  if (group < 1 || group > 65536 || k_group < 1) return HGA_ERR_PARAM;
  const StagedWorkspace w = staged_workspace(shape, group, k_group);
  if (w.stage.pool_pages >= kMaxDim) return HGA_ERR_SHAPE;
  *pool_pages = w.stage.pool_pages;
  *workspace_bytes = w.bytes;
  return HGA_OK;
}

int hga_attend_staged(const hga_shape* shape, const void* Q, const void* K, const void* V,
                      int32_t dtype, const int32_t* group_idx, int32_t k_group, int32_t group,
                      float scale, void* O, float* lse, void* K_pool, void* V_pool,
                      int64_t pool_pages, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !K || !V || !group_idx || !O || !K_pool || !V_pool || !workspace) return HGA_ERR_NULL;
  if (!dtype_ok(dtype)) return HGA_ERR_DTYPE;
  if (group < 1 || group > 65536 || k_group < 1) return HGA_ERR_PARAM;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(K_pool) ||
      !aligned16(V_pool) || !aligned16(workspace))
    return HGA_ERR_LAYOUT;
  const StagedWorkspace w = staged_workspace(shape, group, k_group);
  if (w.stage.pool_pages >= kMaxDim) return HGA_ERR_SHAPE;
  if (pool_pages < w.stage.pool_pages) return HGA_ERR_PARAM;
  if (workspace_bytes < w.bytes) return HGA_ERR_WORKSPACE;
  const int64_t rows = shape->batch * shape->q_heads * shape->n_queries;
  if (rows * w.attend.n_splits >= kMaxDim) return HGA_ERR_SHAPE;
  char* ws = static_cast<char*>(workspace);
  hga::StageArgs sa{};
  sa.K = K;
  sa.V = V;
  sa.K_pool = K_pool;
  sa.V_pool = V_pool;
  sa.group_idx = group_idx;
  sa.B = shape->batch;
  sa.Hq = static_cast<int>(shape->q_heads);
  sa.Hkv = static_cast<int>(shape->kv_heads);
  sa.Nq = static_cast<int>(shape->n_queries);
  sa.T = shape->seq_len;
  sa.D = static_cast<int>(shape->head_dim);
  sa.G = group;
  sa.k_g = k_group;
  sa.marks = reinterpret_cast<uint32_t*>(ws + w.marks);
  sa.block_table = reinterpret_cast<int32_t*>(ws + w.table);
  sa.page_group = reinterpret_cast<int32_t*>(ws + w.pages);
  sa.counts = reinterpret_cast<int32_t*>(ws + w.counts);
  sa.plan = w.stage;
  hipError_t e = hga::launch_stage(sa, dtype, as_stream(stream));
  if (e != hipSuccess) return HGA_ERR_HIP;
  // attention over the pool: B*Hkv sequences of one KV head and r query heads
  // each (the same memory order as [B, Hq, ...]), pages of one group
  const int64_t r = shape->q_heads / shape->kv_heads;
  const hga_shape s2{shape->batch * shape->kv_heads, r, 1, shape->n_queries, shape->seq_len,
                     shape->head_dim};
  hga::KvLayout L{};
  L.paged = 1;
  L.page_tokens = group;
  L.max_pages = static_cast<int>(w.stage.n_g);
  L.n_pages = static_cast<int>(pool_pages);
  L.block_table = sa.block_table;
  const hga::AttendArgs aa = attend_args(&s2, L, Q, K_pool, V_pool, group_idx, k_group, group,
                                         scale, O, lse, workspace, w.attend);
  e = hga::launch_attend(aa, dtype, w.attend, as_stream(stream));
  return e == hipSuccess ? HGA_OK : HGA_ERR_HIP;
}

int hga_decode_step_one_launch_cus(const hga_shape* shape, int32_t dtype, int32_t chunk,
                                   int32_t group, int32_t k_chunk, int32_t k_group,
                                   int32_t compute_units, int32_t* one) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!one) return HGA_ERR_NULL;
  if (!dtype_ok(dtype)) return HGA_ERR_DTYPE;
  if (compute_units < 0) return HGA_ERR_PARAM;
  st = check_route_params(shape, chunk, group, k_chunk, k_group);
  if (st != HGA_OK) return st;
  *one = decode_one_launch(shape, chunk, group, k_chunk, k_group, compute_units) ? 1 : 0;
  return HGA_OK;
}

int hga_decode_step_one_launch(const hga_shape* shape, int32_t dtype, int32_t chunk,
                               int32_t group, int32_t k_chunk, int32_t k_group, int32_t* one) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!one) return HGA_ERR_NULL;
  if (hga::device_cu_count() < 1) return HGA_ERR_HIP;
  return hga_decode_step_one_launch_cus(shape, dtype, chunk, group, k_chunk, k_group,
                                        hga::resident_cu_count(), one);
}

int hga_workspace_check(const void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return HGA_ERR_NULL;
  if (!aligned16(workspace)) return HGA_ERR_LAYOUT;
  if (workspace_bytes < hga::kZeroBytes) return HGA_ERR_WORKSPACE;
  if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return HGA_ERR_HIP;
  int32_t word = 0;
  if (hipMemcpy(&word, static_cast<const char*>(workspace) + hga::kStatusOffset, sizeof(word),
                hipMemcpyDeviceToHost) != hipSuccess)
    return HGA_ERR_HIP;
  return word == 0 ? HGA_OK : HGA_ERR_TIMEOUT;
}

int hga_workspace_reset(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return HGA_ERR_NULL;
  if (!aligned16(workspace)) return HGA_ERR_LAYOUT;
  if (workspace_bytes < hga::kZeroBytes) return HGA_ERR_WORKSPACE;
  return hga::launch_zero_fill(workspace, hga::kZeroBytes, as_stream(stream)) == hipSuccess
             ? HGA_OK
             : HGA_ERR_HIP;
}

int hga_decode_step_ex(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                       const void* K, const void* V, int32_t dtype, float* chunk_mean,
                       float* group_mean, int32_t chunk, int32_t group, int32_t k_chunk,
                       int32_t k_group, float scale, int32_t* chunk_idx, int32_t* group_idx,
                       void* O, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return hga::decode_step_call(shape, layout, Q, K, V, dtype, chunk_mean, group_mean, chunk,
                               group, k_chunk, k_group, scale, chunk_idx, group_idx, O, lse,
                               workspace, workspace_bytes, false, stream);
}

}  // extern "C"

int hga::decode_step_call(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                          const void* K, const void* V, int32_t dtype, float* chunk_mean,
                          float* group_mean, int32_t chunk, int32_t group, int32_t k_chunk,
                          int32_t k_group, float scale, int32_t* chunk_idx, int32_t* group_idx,
                          void* O, float* lse, void* workspace, size_t workspace_bytes,
                          bool clear_first, void* stream) {
  int st = check_shape(shape);
  if (st != HGA_OK) return st;
  if (!Q || !K || !V || !chunk_mean || !group_mean || !group_idx || !O || !workspace)
    return HGA_ERR_NULL;
  if (!dtype_ok(dtype)) return HGA_ERR_DTYPE;
  st = check_route_params(shape, chunk, group, k_chunk, k_group);
  if (st != HGA_OK) return st;
  hga::KvLayout L;
  st = to_layout(layout, shape->seq_len, group, &L);
  if (st != HGA_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
      !aligned16(chunk_mean) || !aligned16(group_mean) || !aligned16(workspace))
    return HGA_ERR_LAYOUT;
  if (workspace_bytes < decode_workspace_bytes(shape, chunk, group, k_chunk, k_group))
    return HGA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  // every argument is valid: from here on the call enqueues work
  if (clear_first && hga::launch_zero_fill(ws, hga::kZeroBytes, as_stream(stream)) != hipSuccess)
    return HGA_ERR_HIP;
  const int cus = hga::resident_cu_count();
  if (!decode_one_launch(shape, chunk, group, k_chunk, k_group, cus)) {
    // refresh + route, then attend
    st = hga_route_fresh_ex(shape, layout, Q, K, dtype, chunk_mean, group_mean, chunk, group,
                            k_chunk, k_group, scale, chunk_idx, group_idx, ws, workspace_bytes,
                            stream);
    if (st != HGA_OK) return st;
    return hga_attend_ex(shape, layout, Q, K, V, dtype, group_idx, k_group, group, scale, O, lse,
                         ws, workspace_bytes, stream);
  }
  const hga::RoutePlan rplan = hga::plan_route(shape->batch, shape->q_heads, shape->kv_heads,
                                               shape->n_queries, shape->seq_len, chunk, group,
                                               k_chunk, k_group);
  const int64_t rows = shape->batch * shape->q_heads * shape->n_queries;
  const hga::AttendPlan aplan = hga::plan_decode_attend(rows, shape->head_dim, k_group, cus);
  hga::RouteArgs ra = route_args(shape, layout, Q, chunk_mean, group_mean, chunk, group, k_chunk,
                                 k_group, scale, chunk_idx, group_idx, ws, rplan);
  ra.K = K;
  ra.kv = L;
  hga::AttendArgs aa = attend_args(shape, L, Q, K, V, group_idx, k_group, group, scale, O, lse,
                                   ws, aplan);
  const hipError_t e = hga::launch_decode_step(ra, aa, aplan, dtype, ws, cus, as_stream(stream));
  return e == hipSuccess ? HGA_OK : HGA_ERR_HIP;
}

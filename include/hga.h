/*
 * libhga: Hierarchical Global Attention (HGA) routed attention for AMD MI355X (gfx950).
 *
 * The method (abstract of "Hierarchical Global Attention (HGA)", arXiv 2606.30709,
 * searcharxiv.com page): a drop-in replacement for dense causal attention with the
 * model's W_Q/W_K/W_V/W_O untouched. For every query head it (1) scores compact
 * RoPE-aware summaries of key chunks and retrieves the relevant chunks, (2) routes
 * only the most relevant groups inside those chunks, and (3) runs exact token-level
 * softmax attention over the retrieved tokens only (about 3% of the context).
 *
 * Readings where the abstract is silent, used by every call below:
 *   - a summary is the mean of the post-RoPE keys of a group or chunk;
 *   - a score is q . summary * scale (scale = 1/sqrt(D) unless given);
 *   - the first chunk and the query's own chunk are always kept, in addition to
 *     the k_chunk best of the other chunks before the query's chunk;
 *   - the k_group best groups are chosen globally among all groups of the kept
 *     chunks whose first position is <= p (forced chunks' groups compete too);
 *   - ties go to the lower index; index lists are ascending and -1 padded;
 *   - query i of Nq sits at position p = T - Nq + i and attends to j <= p.
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major (innermost dimension last, stride 1), and
 *     live in device memory (or host memory the device can address, see
 *     hga_attend). The caller owns every buffer; the library allocates no device
 *     memory and keeps no pointer after a call returns.
 *   - Query head h reads KV head h / (q_heads / kv_heads).
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued in
 *     stream order; nothing synchronises. Results are ready when the stream is.
 *   - Every call returns an hga_status. Arguments are checked on the host before
 *     anything is enqueued; a rejected call enqueues nothing. HGA_ERR_HIP means a
 *     launch failed; faults inside kernels surface at the caller's next
 *     synchronisation, as usual for HIP. Nothing throws, prints or aborts.
 *   - Inputs must be finite (no NaN/Inf in Q, K, V).
 *   - Workspaces: the first hga_workspace_zero_bytes() bytes (4 MiB) of a
 *     workspace hold arrival counters, hand-off words and (in the last 256
 *     bytes) a status word, and must be zero before the workspace's first use
 *     (e.g. allocate it zeroed, or call hga_workspace_reset). Every call leaves
 *     them at zero, so one workspace (large enough for each call) can serve
 *     calls of any shape in turn. Calls that may run concurrently must not
 *     share a workspace. After a call that returned HGA_ERR_HIP, whose kernels
 *     faulted, or after which hga_workspace_check returns HGA_ERR_TIMEOUT, the
 *     region's contents are unspecified: reset it before the workspace's next
 *     use.
 */
#ifndef HGA_H
#define HGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HGA_ABI_VERSION 3

typedef enum hga_status {
  HGA_OK = 0,
  HGA_ERR_NULL = -1,        /* a required pointer is NULL */
  HGA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  HGA_ERR_DTYPE = -3,       /* unknown dtype code */
  HGA_ERR_LAYOUT = -4,      /* a pointer is not 16-byte aligned */
  HGA_ERR_PARAM = -5,       /* chunk/group/k_chunk/k_group/range out of range */
  HGA_ERR_WORKSPACE = -6,   /* workspace smaller than the size query says */
  HGA_ERR_HIP = -7,         /* a HIP call or kernel launch failed */
  HGA_ERR_UNSUPPORTED = -8, /* a valid request this build has no kernel for */
  HGA_ERR_TIMEOUT = -9      /* hga_workspace_check: a bounded wait inside a one-launch decode
                               step on this workspace gave up (its rows were poisoned) */
} hga_status;

typedef enum hga_dtype {
  HGA_F32 = 0,   /* IEEE binary32 */
  HGA_BF16 = 1   /* bfloat16, stored as 16-bit words */
} hga_dtype;

/* Sizes of one attention call. */
typedef struct hga_shape {
  int64_t batch;      /* B  >= 1 sequences */
  int64_t q_heads;    /* Hq >= 1 query heads, a multiple of kv_heads */
  int64_t kv_heads;   /* Hkv >= 1 KV heads */
  int64_t n_queries;  /* Nq, 1 <= Nq <= T: queries per sequence, at positions T-Nq .. T-1 */
  int64_t seq_len;    /* T >= 1 keys per sequence */
  int64_t head_dim;   /* D, 64 or 128 */
} hga_shape;

/* Version of this interface (HGA_ABI_VERSION of the built library). */
int hga_abi_version(void);

/* Size of the zero-at-rest region every workspace begins with (every
 * workspace size query below includes it). */
size_t hga_workspace_zero_bytes(void);

/* Static English text for a status code; never NULL. */
const char* hga_status_str(int status);

/* Number of chunks ceil(T/chunk) and groups ceil(T/group) for a context of
 * seq_len keys. chunk >= 1, group >= 1, chunk % group == 0. Either output may be
 * NULL. */
int hga_summary_counts(int64_t seq_len, int32_t chunk, int32_t group,
                       int64_t* n_chunks, int64_t* n_groups);

/*
 * Step 1, summaries (HGA abstract: compact RoPE-aware chunk summaries; groups are
 * the sub-blocks of a chunk that step 2 routes).
 *   K          [B, Hkv, T, D], dtype `dtype`: post-RoPE keys.
 *   chunk_mean [B, Hkv, ceil(T/chunk), D] f32, written: mean key of each chunk.
 *   group_mean [B, Hkv, ceil(T/group), D] f32, written: mean key of each group.
 * A short last group or chunk is the mean of the keys it has. Accumulation is
 * fp32. chunk % group == 0; chunk / group <= 512; group <= 65536.
 */
int hga_build_summaries(const void* K, int32_t dtype, int64_t batch, int64_t kv_heads,
                        int64_t seq_len, int64_t head_dim, int32_t chunk, int32_t group,
                        float* chunk_mean, float* group_mean, void* stream);

/*
 * Step 1 for a grown or edited cache: recomputes, from K, the summaries of every
 * chunk that holds a token in [t_begin, t_end) and of all groups of those chunks;
 * the rest of chunk_mean/group_mean is left untouched. With 0 <= t_begin < t_end
 * <= T. The recomputed values are bit-identical to what hga_build_summaries
 * writes for them. A decode step that appended key T-1 calls it with
 * [T-1, T). Arguments otherwise as hga_build_summaries.
 */
int hga_update_summaries(const void* K, int32_t dtype, int64_t batch, int64_t kv_heads,
                         int64_t seq_len, int64_t head_dim, int32_t chunk, int32_t group,
                         int64_t t_begin, int64_t t_end,
                         float* chunk_mean, float* group_mean, void* stream);

/* Workspace bytes hga_route needs for this shape and these parameters. */
int hga_route_workspace_size(const hga_shape* shape, int32_t chunk, int32_t group,
                             int32_t k_chunk, int32_t k_group, size_t* bytes);

/*
 * Step 2, two-level routing (HGA abstract: retrieve chunks by summary, then keep
 * only the most relevant groups inside them), for every query head separately.
 *   Q          [B, Hq, Nq, D], dtype `dtype`: post-RoPE queries.
 *   chunk_mean, group_mean: as written by hga_build_summaries for this T.
 *   k_chunk >= 0 chunks kept by score besides the first and the query's own;
 *   k_group >= 1 groups kept. Limits: ceil(T/chunk) <= 4098,
 *   min(k_chunk + 2, ceil(T/chunk)) <= 1024 and
 *   min(k_chunk + 2, ceil(T/chunk)) * (chunk/group) <= 4096 (else
 *   HGA_ERR_UNSUPPORTED).
 *   scale      score scale; <= 0 means 1/sqrt(D).
 *   chunk_idx  [B, Hq, Nq, k_chunk + 2] int32 or NULL, written: kept chunk ids,
 *              ascending, -1 padded.
 *   group_idx  [B, Hq, Nq, k_group] int32, written: kept group ids, ascending,
 *              -1 padded.
 * Scores are fp32; equal fp32 scores go to the lower index.
 */
int hga_route(const hga_shape* shape, const void* Q, int32_t dtype,
              const float* chunk_mean, const float* group_mean, int32_t chunk, int32_t group,
              int32_t k_chunk, int32_t k_group, float scale,
              int32_t* chunk_idx, int32_t* group_idx,
              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes hga_attend needs for this shape and these parameters. */
int hga_attend_workspace_size(const hga_shape* shape, int32_t group, int32_t k_group,
                              size_t* bytes);

/*
 * Step 3, exact attention over the routed tokens (HGA abstract: exact
 * token-level attention over the retrieved set only).
 *   Q         [B, Hq, Nq, D]; K, V [B, Hkv, T, D]; all of dtype `dtype`.
 *             K and V may live in pinned host memory the device can address
 *             (hipHostMalloc); the kernel then reads only the routed groups.
 *   group_idx [B, Hq, Nq, k_group] int32 group ids in [0, ceil(T/group)), as
 *             hga_route writes them; -1 (and any id outside that range) is
 *             ignored. Each id must appear at most once per row.
 *   O         [B, Hq, Nq, D] of dtype `dtype`, written:
 *             O = sum_j softmax_j(scale * q.k_j) v_j over j in the listed groups,
 *             j <= p, with fp32 accumulation.
 *   lse       [B, Hq, Nq] f32 or NULL, written: natural-log log-sum-exp of the
 *             scaled logits over the same tokens.
 *   scale     <= 0 means 1/sqrt(D).
 * A row with no token gets O = 0 and lse = -inf.
 */
int hga_attend(const hga_shape* shape, const void* Q, const void* K, const void* V,
               int32_t dtype, const int32_t* group_idx, int32_t k_group, int32_t group,
               float scale, void* O, float* lse,
               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Ragged and paged K/V (batched serving).
 *
 * The same three steps over a batch whose sequences hold different numbers of
 * keys, with K/V either dense [B, Hkv, T, D] (T = capacity) or in a pool of
 * pages addressed through a block table. Sequence b holds seq_lens[b] keys
 * (clamped to [0, T]); its Nq queries sit at positions seq_lens[b]-Nq ..
 * seq_lens[b]-1 (queries at negative positions route to nothing: -1 indices,
 * O = 0, lse = -inf). Summaries stay [B, Hkv, ceil(T/chunk), D]; entries past a
 * sequence's last chunk are not written and never read by routing.
 * ------------------------------------------------------------------------ */
typedef enum hga_kv_kind {
  HGA_KV_DENSE = 0,  /* K, V are [B, Hkv, T, D] */
  HGA_KV_PAGED = 1   /* K, V are page pools [n_pages, Hkv, page_tokens, D] */
} hga_kv_kind;

typedef struct hga_kv_layout {
  int32_t kind;                /* hga_kv_kind */
  int32_t page_tokens;         /* paged: tokens per page, a multiple of `group` */
  int32_t max_pages;           /* paged: columns of block_table, >= ceil(T / page_tokens) */
  int32_t n_pages;             /* paged: pages in the pool; a page id outside [0, n_pages)
                                  holds no keys: attention skips the groups on it (their
                                  tokens count as absent), and the summaries take its
                                  tokens as zero keys (a group mean of 0) */
  const int32_t* block_table;  /* paged: [B, max_pages] int32 page ids, device memory;
                                  token t of sequence b is row t % page_tokens of page
                                  block_table[b][t / page_tokens] */
  const int32_t* seq_lens;     /* [B] int32 keys per sequence, device memory; NULL: all T */
} hga_kv_layout;

/* hga_build_summaries over a ragged/paged cache (layout may be NULL = dense, all T). */
int hga_build_summaries_ex(const void* K, int32_t dtype, const hga_kv_layout* layout,
                           int64_t batch, int64_t kv_heads, int64_t seq_len, int64_t head_dim,
                           int32_t chunk, int32_t group, float* chunk_mean, float* group_mean,
                           void* stream);

/* Recomputes, for every sequence, the summaries of the chunks holding its
 * newest `newest` keys (1 <= newest <= seq_len) and of all their groups: the
 * decode-step refresh after each sequence appended `newest` keys. */
int hga_update_summaries_ex(const void* K, int32_t dtype, const hga_kv_layout* layout,
                            int64_t batch, int64_t kv_heads, int64_t seq_len, int64_t head_dim,
                            int32_t chunk, int32_t group, int64_t newest,
                            float* chunk_mean, float* group_mean, void* stream);

/* hga_route with per-sequence lengths (only layout->seq_lens is used; NULL
 * layout = all T). Workspace as hga_route_workspace_size. */
int hga_route_ex(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                 int32_t dtype, const float* chunk_mean, const float* group_mean, int32_t chunk,
                 int32_t group, int32_t k_chunk, int32_t k_group, float scale,
                 int32_t* chunk_idx, int32_t* group_idx,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Decode-step form of step 1 + step 2: hga_update_summaries_ex(newest = Nq)
 * followed by hga_route_ex, with the same results bit for bit. For small
 * batches (B*Hq*Nq <= 1024, Nq <= chunk, chunk/group <= 16, the routing
 * state within 64 KiB of LDS, not the MFMA prefill case) it runs as one
 * launch: each routing workgroup recomputes the newest chunks of its sequence
 * from K, writes them to chunk_mean/group_mean
 * and scores with them; otherwise it enqueues the two calls. K is the cache the
 * layout describes. Workspace as hga_route_workspace_size. */
int hga_route_fresh_ex(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                       const void* K, int32_t dtype, float* chunk_mean, float* group_mean,
                       int32_t chunk, int32_t group, int32_t k_chunk, int32_t k_group,
                       float scale, int32_t* chunk_idx, int32_t* group_idx,
                       void* workspace, size_t workspace_bytes, void* stream);

/* hga_attend over a ragged/paged cache (layout may be NULL = dense, all T).
 * Paged K and V are page pools; group ids index the sequence's logical
 * tokens. Workspace as hga_attend_workspace_size. */
int hga_attend_ex(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                  const void* K, const void* V, int32_t dtype, const int32_t* group_idx,
                  int32_t k_group, int32_t group, float scale, void* O, float* lse,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Pool pages and workspace bytes hga_attend_staged needs for this shape. */
int hga_attend_staged_sizes(const hga_shape* shape, int32_t group, int32_t k_group,
                            int64_t* pool_pages, size_t* workspace_bytes);

/*
 * Step 3 for K/V in memory the device reads slowly, such as pinned host memory
 * (HGA abstract: the full K/V need not sit in device memory; only the routed
 * tokens are fetched). The r*Nq query rows of one (sequence, KV head) share
 * much of their routing, so the routed groups are first deduplicated per
 * (sequence, KV head) and each is copied once into a device pool; attention
 * then reads the pool. O and lse equal hga_attend's on the same arguments,
 * bit for bit.
 *   Q, K, V, group_idx, O, lse, scale: as hga_attend (K, V dense
 *             [B, Hkv, T, D], in any memory the device can address).
 *   K_pool, V_pool: device memory of pool_pages pages of [group, D] elements
 *             of `dtype` each, pool_pages >= the count hga_attend_staged_sizes
 *             gives (B*Hkv*min(ceil(T/group), r*Nq*k_group)); scratch.
 *   workspace: hga_attend_staged_sizes bytes; its zero region zero, as always.
 * The bytes read from K and V are the distinct routed groups' (what
 * crosses the host link), not every row's.
 */
int hga_attend_staged(const hga_shape* shape, const void* Q, const void* K, const void* V,
                      int32_t dtype, const int32_t* group_idx, int32_t k_group, int32_t group,
                      float scale, void* O, float* lse, void* K_pool, void* V_pool,
                      int64_t pool_pages, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Workspace bytes hga_decode_step_ex needs. As for every call here, the
 * workspace's zero region must be zero before its first use and is left
 * zero; the rest is scratch. */
int hga_decode_step_workspace_size(const hga_shape* shape, int32_t chunk, int32_t group,
                                   int32_t k_chunk, int32_t k_group, size_t* bytes);

/* Whether hga_decode_step_ex runs these arguments as one launch on the
 * current device: *one = 1, else 0 (the calls it then enqueues are
 * hga_route_fresh_ex and hga_attend_ex). The one-launch form needs every one
 * of its workgroups resident at once, one per compute unit: it is chosen only
 * when the grid fits the device's compute units (queried once per device),
 * and never when a CU mask (HSA_CU_MASK or ROC_GLOBAL_CU_MASK) is set in the
 * environment. HGA_ERR_HIP if there is no current device. */
int hga_decode_step_one_launch(const hga_shape* shape, int32_t dtype, int32_t chunk,
                               int32_t group, int32_t k_chunk, int32_t k_group, int32_t* one);

/* The same decision for a device whose workgroups can hold `compute_units`
 * compute units at once (>= 0; 0: never one launch). Needs no device. */
int hga_decode_step_one_launch_cus(const hga_shape* shape, int32_t dtype, int32_t chunk,
                                   int32_t group, int32_t k_chunk, int32_t k_group,
                                   int32_t compute_units, int32_t* one);

/*
 * Status of a workspace after the work enqueued on `stream`: synchronises the
 * stream, then reads the workspace's status word. HGA_OK if every bounded wait
 * of the one-launch decode steps on it completed; HGA_ERR_TIMEOUT if one gave
 * up (its rows got NaN in O and lse and -1 ids). The flag is sticky: until the
 * workspace is reset, every later one-launch decode step on it reads no
 * hand-off word (late stores of the step that gave up may have left some) and
 * poisons its rows the same way, while still refreshing the summaries.
 * Waits give up only if the step's workgroups are not all resident at once
 * (a concurrent kernel holding compute units the step was planned for).
 * workspace_bytes >= hga_workspace_zero_bytes(). Not for use during stream
 * capture (it synchronises).
 */
int hga_workspace_check(const void* workspace, size_t workspace_bytes, void* stream);

/* Zeroes the workspace's zero region (status word included) on `stream`, with
 * a kernel (no memset, so the call can be captured in a graph). */
int hga_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step, all three HGA steps (abstract: summaries, routing by
 * summary, exact attention over the routed tokens): the same results as
 * hga_route_fresh_ex followed by hga_attend_ex on the same arguments
 * (chunk_idx, group_idx, chunk_mean and group_mean bit for bit; O and lse to
 * fp32 rounding, the attention's partial sums being grouped differently).
 *   Q [B, Hq, Nq, D]; K, V as the layout describes (NULL = dense, all T);
 *   chunk_mean, group_mean: the summaries, whose chunks holding each
 *   sequence's newest Nq keys are recomputed from K and written;
 *   chunk_idx (or NULL), group_idx, O, lse (or NULL): written as by
 *   hga_route_ex and hga_attend_ex.
 * For small batches (hga_decode_step_one_launch: every workgroup of the step
 * fits the device at once, one per CU, and the rows' scores fit the
 * workspace's zero region) the call is one launch: every workgroup scores a
 * share of one KV head's summaries against all of its query rows and writes
 * the scores into the zero region as words that are never zero; then it polls
 * its own row's words until all have arrived (a bounded wait; a row whose
 * scores do not all arrive in time gets NaN in O and lse and -1 ids, and the
 * workspace's status word records it: see hga_workspace_check), selects, and
 * attends to its share of the row's groups. The workgroup that finishes a row
 * zeroes the row's words. Otherwise the two calls are enqueued. Calls that
 * share a workspace must not overlap, and no other kernel should hold the
 * device's compute units while a one-launch step runs.
 */
int hga_decode_step_ex(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                       const void* K, const void* V, int32_t dtype, float* chunk_mean,
                       float* group_mean, int32_t chunk, int32_t group, int32_t k_chunk,
                       int32_t k_group, float scale, int32_t* chunk_idx, int32_t* group_idx,
                       void* O, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * hga_decode_step_ex for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, with the same results, whose scratch is a fixed
 * 16 MiB array in the library's own device memory instead of a caller
 * workspace. The call allocates nothing.
 *   Arguments as hga_decode_step_ex, without workspace and workspace_bytes.
 *   reset      non-zero: clear the scratch's zero region first (in stream
 *              order), as after a step whose bounded wait gave up (its rows
 *              NaN; every later step on the scratch stays poisoned until a
 *              reset). The first call on each device clears it by itself.
 * HGA_ERR_WORKSPACE if the step needs more scratch than the array holds
 * (hga_decode_step_workspace_size > 16 MiB; e.g. more than 42 sequences at a
 * 64K context with 32 query heads): use hga_decode_step_ex then. Each device
 * the library runs on holds its own array until the process ends. Every call
 * on one device shares that device's array, which keeps the last call's
 * contents: calls that overlap on one device (other streams or threads) race.
 */
int hga_decode_step_noalloc(const hga_shape* shape, const hga_kv_layout* layout, const void* Q,
                            const void* K, const void* V, int32_t dtype, float* chunk_mean,
                            float* group_mean, int32_t chunk, int32_t group, int32_t k_chunk,
                            int32_t k_group, float scale, int32_t* chunk_idx, int32_t* group_idx,
                            void* O, float* lse, int32_t reset, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HGA_H */

/*
 * resa.h: C ABI of libresa.so, the MI355X (gfx950) hot path of Rectified Sparse
 * Attention (ReSA): block-sparse decoding over a paged KV cache with Quest-style
 * block descriptors, group block-sparse selection (GBSA), and periodic dense
 * rectification.
 *
 * Sources: "Rectified Sparse Attention" (arXiv 2506.04108), abstract; Pith review
 * of "Rectified Sparse Attention", sections "What carries the argument", "The
 * reading", referee report major comment 1 (the paper's Eq. 5 and Eq. 6) and
 * minor comment 3 (Eq. 2), "Assumptions & free parameters".
 *
 * Conventions (all entry points):
 *  - Pointers are device pointers unless marked (host). Arrays are row-major with
 *    the head dimension innermost. The caller owns every buffer, the workspace
 *    included; the library never allocates or frees device memory (the one
 *    exception, resa_sparse_decode_noalloc's scratch array, is a static device
 *    array loaded with the library, not an allocation).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronises with the host.
 *  - Alignment: the cache's k_pages, v_pages and desc, and every q, k_new,
 *    v_new, out and workspace pointer, must be 16-byte aligned; block_table,
 *    seq_lens, idx and count 4-byte aligned (allocations from hipMalloc, and
 *    their rows, are). A misaligned pointer returns RESA_ERR_INVALID.
 *  - Arguments are validated on the host before any launch. A bad argument
 *    returns RESA_ERR_INVALID or RESA_ERR_UNSUPPORTED and launches nothing; a
 *    failed launch returns RESA_ERR_HIP. resa_last_error() then gives a message.
 *  - Device-side preconditions (seq_lens[b] <= max_seq_len, block_table entries
 *    in [0, num_pages) for every block a sequence holds, seq_lens[b] >= 1 for
 *    selection and decoding, f <= seq_lens[b] for rectification) are the
 *    caller's; the library as normally built does not check them. A build with
 *    RESA_DEBUG_CHECKS defined checks them on the device: every call then waits
 *    for its stream and returns RESA_ERR_INVALID if one failed (a call under
 *    HIP graph capture leaves the report to the next uncaptured call).
 *  - Workspaces: each call takes a caller-owned workspace of at least the size
 *    its *_workspace_size() function returns. Its contents on entry do not
 *    matter and are dead on return, so one workspace may serve all calls issued
 *    in order on one stream. Calls that may run concurrently need separate
 *    workspaces.
 *  - The library holds no mutable state apart from the thread-local error text
 *    (and resa_sparse_decode_noalloc's scratch array), so calls on different
 *    streams from different host threads are safe as long as they do not share
 *    output buffers or workspace.
 */
#ifndef RESA_H
#define RESA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RESA_OK = 0,
  RESA_ERR_INVALID = 1,     /* NULL pointer, bad size, inconsistent shape */
  RESA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, group size, length */
  RESA_ERR_WORKSPACE = 3,   /* workspace smaller than the *_workspace_size() call says */
  RESA_ERR_HIP = 4          /* a HIP launch failed */
} resa_status;

typedef enum { RESA_FP32 = 0, RESA_BF16 = 1 } resa_dtype;

/*
 * The paged KV cache. A page holds one block of b = 16 consecutive tokens of one
 * sequence, for every KV head. Sequence b's token t lives in page
 * block_table[b * max_blocks_per_seq + t / 16], slot t % 16.
 *
 *   k_pages          : [num_pages][num_kv_heads][16][head_dim]   (dtype), token-major
 *   v_pages          : [num_pages][num_kv_heads][head_dim][16]   (dtype), channel-major:
 *                      V[t][c] of the page is at [..][c][t % 16]
 *   desc             : [num_pages][num_kv_heads][2][head_dim]    (dtype)
 *                      [..][0][c] = min over the block's valid tokens of K[., c],
 *                      [..][1][c] = max (the Quest-style block descriptor of
 *                      Pith "What carries the argument"; exact, no rounding)
 *   block_table      : [batch][max_blocks_per_seq] int32 page ids
 *   seq_lens         : [batch] int32, tokens held, the newest token included
 *
 * dtype: q, K, V, descriptors and outputs share it. head_dim in {64, 128};
 * num_q_heads = G * num_kv_heads with group size G in {1, 2, 4, 8};
 * block_size must be 16 (the page size is the selection block).
 * Limits of the library, RESA_ERR_UNSUPPORTED beyond them: max_blocks_per_seq
 * <= 32768 (524,288 tokens per sequence) and num_kv_heads * head_dim <= 4096.
 */
typedef struct resa_cache {
  int32_t dtype;              /* resa_dtype */
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;         /* must be 16 */
  int32_t num_pages;
  int32_t max_blocks_per_seq;
  int32_t max_seq_len;        /* (host) upper bound on every seq_lens[b] */
  void* k_pages;
  void* v_pages;
  void* desc;
  const int32_t* block_table;
  const int32_t* seq_lens;
} resa_cache;

/*
 * Selection parameters. Eq. 5 (Pith referee report, major comment 1) with its
 * ratio read as an explicit active-block ratio r:
 *   M = ceil(L / 16),  n = min(M, max(n_min, ceil(M * r)))   (IEEE double)
 * n_local: the newest blocks (the partial current block included) that are
 * always selected and count toward n (Pith "Assumptions & free parameters").
 */
typedef struct resa_select_params {
  int32_t n_min;    /* >= 1 */
  int32_t n_local;  /* >= 0 */
  double r;         /* in (0, 1] */
} resa_select_params;

/* (host) Largest n any sequence can have: n at M = ceil(max_seq_len / 16).
 * This is the row stride of idx. Returns -1 on a bad argument. */
int32_t resa_n_cap(const resa_cache* cache, const resa_select_params* params);

/* (host) Workspace bytes each call needs for this cache (0 on a bad argument). */
size_t resa_select_workspace_size(const resa_cache* cache);
size_t resa_decode_workspace_size(const resa_cache* cache, int32_t n_cap);
size_t resa_rectify_workspace_size(const resa_cache* cache, int32_t f);

/*
 * Write new tokens into the cache and bring the block descriptors up to date
 * (block statistics, Pith "What carries the argument").
 *
 * n_new >= 1: for every sequence b, positions [seq_lens[b] - n_new, seq_lens[b])
 *   (seq_lens already counts them) receive k_new[b][i], v_new[b][i]
 *   ([batch][n_new][num_kv_heads][head_dim], dtype) unless k_new and v_new are
 *   both NULL (the cache already holds them). Then the descriptor of every block
 *   holding one of those positions is recomputed over its valid tokens. This is
 *   the per-step append (n_new = 1).
 * n_new == 0: rebuild the descriptor of every block of every sequence from the
 *   cache (after a prefill, or when resuming from saved K/V). k_new and v_new
 *   must be NULL.
 * Positions below 0 (n_new > seq_lens[b]) are skipped.
 */
resa_status resa_update_descriptors(const resa_cache* cache, const void* k_new, const void* v_new,
                                    int32_t n_new, void* stream);

/*
 * GBSA block selection (Pith "What carries the argument"). For every sequence b
 * and KV head g: the group's query heads g*G .. g*G+G-1 are pooled into their
 * mean q_bar (summed in head order in float64, then divided by G); every block j
 * of the sequence is scored with the Quest upper bound
 *   s_j = sum_c max(q_bar_c * kmin_jc, q_bar_c * kmax_jc)   (float64, unscaled)
 * and the selection is the min(n_local, n) newest blocks plus the highest-scoring
 * other blocks (ties: lower index first) up to n blocks in total.
 *
 *   q     : [batch][num_q_heads][head_dim] (dtype), the decode queries
 *   idx   : [batch][num_kv_heads][n_cap] int32 out; row (b, g) holds the n_b
 *           selected block indices (logical, 0 .. M_b - 1) in ascending order;
 *           entries past n_b are left as they were
 *   count : [batch] int32 out; count[b] = n_b
 *   n_cap : row stride of idx, >= resa_n_cap(cache, params)
 *   ws    : >= resa_select_workspace_size(cache) bytes
 */
resa_status resa_select_blocks(const resa_cache* cache, const void* q, const resa_select_params* params,
                               int32_t* idx, int32_t* count, int32_t n_cap, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * One decode step's cache append and block selection (Pith "What carries the
 * argument": the newest token's key enters its block's statistics before the
 * step's selection). The result is exactly that of
 *   resa_update_descriptors(cache, k_new, v_new, 1, stream);
 *   resa_select_blocks(cache, q, params, idx, count, n_cap, ws, ws_bytes, stream);
 * (k_new, v_new: [batch][1][num_kv_heads][head_dim], or both NULL when the cache
 * already holds the new token). With params->n_local >= 1 the newest block is
 * always selected and never scored, so the append runs inside the scoring
 * launch; with n_local == 0 the two run one after the other. Arguments, output
 * layout, workspace and errors are those of the two calls above.
 */
resa_status resa_append_select(const resa_cache* cache, const void* k_new, const void* v_new, const void* q,
                               const resa_select_params* params, int32_t* idx, int32_t* count, int32_t n_cap,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Block-sparse decoding (Eq. 2, Pith referee report minor comment 3): head h of
 * sequence b attends to exactly the valid tokens of the blocks its group g = h / G
 * selected,
 *   out[b][h] = softmax_t(scale * q[b][h] . K[t]) V[t],   t in the selected blocks,
 * with fp32 accumulation (split over the key axis, then an exact log-sum-exp merge).
 *
 *   q     : [batch][num_q_heads][head_dim] (dtype)
 *   idx, count, n_cap : as written by resa_select_blocks (any sorted or unsorted
 *           set of distinct valid block indices is accepted)
 *   scale : logit scale, 1/sqrt(head_dim) in the usual case
 *   out   : [batch][num_q_heads][head_dim] (dtype), rounded to nearest even
 *   ws    : >= resa_decode_workspace_size(cache, n_cap) bytes
 */
resa_status resa_sparse_decode(const resa_cache* cache, const void* q, const int32_t* idx,
                               const int32_t* count, int32_t n_cap, float scale, void* out, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * resa_sparse_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation): the same kernels and the same result, bit for bit, with
 * the split partials in a scratch array of 16 MiB that the library holds in
 * device memory on each GPU it runs on, until the process ends. Arguments as
 * for resa_sparse_decode.
 *  - Calls a configuration whose decode workspace would exceed 16 MiB
 *    (resa_decode_workspace_size) rejected with RESA_ERR_UNSUPPORTED.
 *  - Runs on the current device; a non-NULL stream must belong to it
 *    (RESA_ERR_INVALID otherwise). The first call on a device looks the
 *    scratch array up (hipGetSymbolAddress); make that call outside graph
 *    capture.
 *  - Every call on a GPU shares that GPU's scratch array: calls that may
 *    overlap on one GPU (different streams, or threads) race, so issue them in
 *    order on one stream. The partials need no clearing: a call writes every
 *    slot it reads.
 *  - Allocates nothing: no hipMalloc or hipFree, no allocating library call.
 */
resa_status resa_sparse_decode_noalloc(const resa_cache* cache, const void* q, const int32_t* idx,
                                       const int32_t* count, int32_t n_cap, float scale, void* out,
                                       void* stream);

/*
 * Dense rectification (Pith "What carries the argument", "The reading"): the f
 * newest positions [L_b - f, L_b) of every sequence (L_b = seq_lens[b]) are
 * overwritten with the re-encoded k_new, v_new, the descriptors of the touched
 * blocks are recomputed, and row i of every head attends causally over the
 * updated cache:
 *   out[b][i][h] = softmax_{t <= L_b - f + i}(scale * q[b][i][h] . K[t]) V[t].
 *
 *   q            : [batch][f][num_q_heads][head_dim] (dtype)
 *   k_new, v_new : [batch][f][num_kv_heads][head_dim] (dtype)
 *   f            : 1 .. 1024, and f <= seq_lens[b] for every b
 *   out          : [batch][f][num_q_heads][head_dim] (dtype)
 *   ws           : >= resa_rectify_workspace_size(cache, f) bytes
 */
resa_status resa_rectify(const resa_cache* cache, const void* q, const void* k_new, const void* v_new,
                         int32_t f, float scale, void* out, void* ws, size_t ws_bytes, void* stream);

/* Message for the last non-OK status returned on this host thread ("" if none). */
const char* resa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RESA_H */

/*
 * yoco.h -- C ABI of the YOCO cross-decoder hot path on AMD MI355X (gfx950).
 *
 * YOCO ("You Only Cache Once") splits a decoder into a self-decoder that
 * writes one shared, token-level K/V cache and a cross-decoder whose layers
 * each issue their own query and all read that same cache.  This library
 * implements the three steps of the cross-decoder side of one inference step:
 *
 *   yoco_kv_append   K^ = RMSNorm(M) W_K, V^ = RMSNorm(M) W_V for every
 *                    scheduled token, written once into the paged cache.
 *   yoco_gather_last keep only each request's last scheduled token.
 *   yoco_cross_attn  one cross layer: each request's query heads attend to
 *                    the request's whole context in the shared paged cache.
 *
 * and the general forms the same pages call for:
 *
 *   yoco_gather_logits      any number of rows per request (the logits
 *                           positions), with the cross-decoder's
 *                           query_start_loc rebuilt on the device.
 *   yoco_cross_attn_varlen  several query rows per request (causal, aligned
 *                           to the end of the context) and an optional
 *                           sliding window.
 *
 * Conventions shared by every call
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; every call is asynchronous on
 *     `stream` (a hipStream_t; NULL means the null stream) and may be
 *     captured in a HIP graph.  A call that returns YOCO_OK has only
 *     enqueued work.
 *   - Scalar arguments are validated on the host BEFORE anything is
 *     launched; on failure nothing is enqueued and a status code is returned
 *     (yoco_last_error_message() gives the reason, per calling thread).
 *   - Device-side index data (cu_seqlens, slot_mapping, block_table,
 *     seq_lens) is not validated: the stated preconditions are the caller's.
 *     Kernels never read or write outside the buffers the arguments describe
 *     even when an index breaks them (such entries are skipped); the numbers
 *     produced for the affected rows are then unspecified.
 *   - Paged cache layout: two tensors, K and V, each
 *         [num_blocks][num_kv_heads][block_size][head_dim]
 *     row-major in the cache dtype.  Token j of a request lives in physical
 *     block block_table[r][j / block_size], row j % block_size; a slot number
 *     s names block s / block_size, row s % block_size.
 *   - dtype: YOCO_DTYPE_F32 (fp32 everywhere) or YOCO_DTYPE_BF16 (bf16
 *     cache, queries, activations and weights; fp32 accumulation; attention
 *     output is always fp32).
 *
 * The operations are defined on these pages (cited by title and section):
 *   [vLLM] "You Only Cache Once, in vLLM", section "Implementation in vLLM".
 *   [YOCO] "YOCO_论文与推理数据流详解", sections 3, 4.1-4.2, 7.4, 9, 10.3, 10.4, 13.
 *   [KV]   "KV cache memory systems", sections "Cache contents" and
 *          "Contiguous allocation wastes capacity".
 *   [Gemma] "You Only Cache Once, in vLLM", section "Gemma 3n": cross layers
 *          that reuse a sliding-window layer's cache.
 */
#ifndef YOCO_H_
#define YOCO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define YOCO_ABI_VERSION 7

typedef enum yoco_status {
  YOCO_OK = 0,
  YOCO_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, inconsistent shapes */
  YOCO_ERR_UNSUPPORTED = 2,        /* a valid shape the library has no kernel for */
  YOCO_ERR_WORKSPACE_TOO_SMALL = 3,
  YOCO_ERR_HIP = 4                 /* the HIP runtime refused a launch */
} yoco_status_t;

/* YOCO_DTYPE_FP8_E4M3 is a cache dtype only: one byte per element in the
 * FP8 E4M3 format (finite-only variant: bias 7, 0x7F/0xFF NaN, largest 448),
 * plus one fp32 scale per (token, KV head) for K and one for V, laid out
 * [num_blocks][num_kv_heads][block_size]; an element means code * scale. */
typedef enum yoco_dtype { YOCO_DTYPE_F32 = 0, YOCO_DTYPE_BF16 = 1, YOCO_DTYPE_FP8_E4M3 = 2 } yoco_dtype_t;

/* yoco_cross_attn flag: walk the (request, KV head, partition) work items in
 * reverse order (when contexts end in tail pieces, see partition_tokens:
 * the full partitions and, separately, the pieces, which still come last).
 * Alternating it between consecutive cross layers
 * makes the first blocks a layer reads the last ones the previous layer read,
 * which may still sit in the GPU's last-level cache (the kernels read K^/V^
 * rows with a streaming hint that mostly keeps them out of it).  Results are
 * bit-identical either way. */
#define YOCO_FLAG_REVERSE_ORDER 1u

/* yoco_cross_attn and yoco_cross_attn_varlen flag: run the vector-ALU kernel
 * even where the matrix-core kernel is the default (an FP8 cache, several
 * query rows per request, or a bf16 cache at head_dim 256 with partitions of
 * at least 512 tokens; yoco_cross_attn_kernel tells which).  Same results
 * within the attention tolerance; for comparisons. */
#define YOCO_FLAG_VECTOR_KERNEL 2u

/* The first YOCO_CROSS_ATTN_QUEUE_BYTES bytes of a yoco_cross_attn workspace
 * are the work-queue counters of its persistent schedule: they must be zero
 * before the first call with that workspace, and every call leaves them zero
 * again. */
#define YOCO_CROSS_ATTN_QUEUE_BYTES 2048

/*
 * Precondition checks (debugging aid).
 *
 * The calls do not validate device-side index data (see the conventions
 * above).  With validation on -- YOCO_VALIDATE=1 (any value but 0) in the
 * environment when the library first asks, or yoco_set_validation(1) --
 * every call copies its index arrays to the host, synchronises `stream`,
 * checks them with the functions below and returns YOCO_ERR_INVALID_ARGUMENT
 * (yoco_last_error_message() names the first violation) before launching
 * anything.  Calls then wait for the GPU, so this is for debugging only; on
 * a stream being captured into a graph the checks are skipped.
 *
 * The checks take HOST arrays and return YOCO_OK or YOCO_ERR_INVALID_ARGUMENT:
 *   yoco_validate_offsets         cu_seqlens / query_start_loc [num_reqs+1]:
 *                                 non-decreasing, within [0, num_rows].
 *   yoco_validate_slots           slot_mapping [num_tokens]: every
 *                                 non-negative slot < num_blocks*block_size,
 *                                 no slot twice.
 *   yoco_validate_block_table     seq_lens [num_seqs] in [0, max_seq_len] and
 *                                 within a table row; every block the call
 *                                 reads (from the first position any query of
 *                                 the request sees, with query_start_loc and
 *                                 window as in yoco_cross_attn_varlen; NULL
 *                                 query_start_loc = one row per request) in
 *                                 [0, num_blocks); query_start_loc checked as
 *                                 offsets of num_rows rows.
 *   yoco_validate_logits_indices  non-decreasing, each inside the batch's rows
 *                                 [query_start_loc[0], query_start_loc[R]).
 *   yoco_validate_state_indices   each slot < num_slots (negative = none), no
 *                                 slot twice.
 * Pages: "KV cache memory systems", section "Contiguous allocation wastes
 * capacity" (each logical block resolves through the block table to a
 * physical page); "You Only Cache Once, in vLLM", section "Implementation in
 * vLLM" (the metadata: offsets of consecutive rows, per-token slots, logits
 * positions in order).
 */
void yoco_set_validation(int32_t enabled);
int32_t yoco_validation_enabled(void);
int32_t yoco_validate_offsets(const int32_t* offsets, int32_t num_reqs, int64_t num_rows);
int32_t yoco_validate_slots(const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks, int32_t block_size);
int32_t yoco_validate_block_table(const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
                                  const int32_t* seq_lens, int32_t max_seq_len, int32_t num_blocks,
                                  int32_t block_size, const int32_t* query_start_loc, int32_t num_rows,
                                  int32_t window);
int32_t yoco_validate_logits_indices(const int32_t* logits_indices, int32_t num_indices,
                                     const int32_t* query_start_loc, int32_t num_reqs, int64_t num_tokens);
int32_t yoco_validate_state_indices(const int32_t* state_indices, int32_t num_reqs, int32_t num_slots);

/* Version of this ABI (YOCO_ABI_VERSION). */
int32_t yoco_abi_version(void);

/* Static text for a status code. */
const char* yoco_status_string(int32_t status);

/* Reason for the most recent non-OK status returned on the calling thread
 * (empty string if none). */
const char* yoco_last_error_message(void);

/*
 * yoco_gather_last -- one row per request: its last scheduled token.
 *
 * [vLLM] "Implementation in vLLM": within one mixed prefill/decode step the
 * cross-decoder needs only the last scheduled token of each request, so its
 * batch collapses to one row per request.  [YOCO] section 7.4: only the last
 * prompt position enters the cross-decoder at prefill; at decode it is the
 * new token.
 *
 *   hidden      [num_tokens][row_bytes], token-major, row stride row_bytes.
 *               Rows are copied bit for bit (any element type).
 *   num_tokens  rows in hidden (graph-padding rows included), >= 0.
 *   row_bytes   bytes per row; must be a positive multiple of 16, and hidden
 *               and out must be 16-byte aligned.
 *   cu_seqlens  int32 [num_reqs + 1]: request r owns rows
 *               cu_seqlens[r] .. cu_seqlens[r+1]-1.  Precondition:
 *               non-decreasing, within [0, num_tokens].
 *   out         [num_reqs][row_bytes]: out[r] = hidden[cu_seqlens[r+1]-1].
 *               A request with no rows (or whose row index falls outside
 *               [0, num_tokens)) gets a row of zero bytes.
 *   out_index   optional int32 [num_reqs] (may be NULL): the row taken, or -1.
 *
 * Errors: YOCO_ERR_INVALID_ARGUMENT for null pointers (other than
 * out_index), negative counts, bad row_bytes or misalignment.  num_reqs == 0
 * is a no-op.
 */
int32_t yoco_gather_last(const void* hidden, int64_t num_tokens, int64_t row_bytes,
                         const int32_t* cu_seqlens, int32_t num_reqs,
                         void* out, int32_t* out_index, void* stream);

/*
 * yoco_kv_append -- the shared K/V projection, once per token, into the cache.
 *
 * [YOCO] section 3 (architecture flowchart) and section 10.3: from the
 * self-decoder output M, K^ = LN(M) W_K and V^ = LN(M) W_V are computed once
 * per token and appended to the single global cache that every cross layer
 * reads; nothing is appended per cross layer.  LN is read as RMSNorm:
 *     xhat = x / sqrt(mean(x^2) + eps) * rms_weight
 *     K^_t = W_K xhat_t,  V^_t = W_V xhat_t      (no bias)
 * and K^_t, V^_t (each [num_kv_heads][head_dim]) are written to slot
 * slot_mapping[t] of the K and V caches.  [vLLM] "Implementation in vLLM":
 * slot_mapping is the per-token slot list of the attention metadata.
 *
 *   dtype        YOCO_DTYPE_F32 or YOCO_DTYPE_BF16: type of x, rms_weight,
 *                w_k, w_v and the cache.
 *   x            [num_tokens][hidden] row-major.
 *   rms_weight   [hidden].
 *   eps          added to mean(x^2) inside the square root, >= 0.
 *   w_k, w_v     [num_kv_heads*head_dim][hidden] row-major (output features
 *                by input features).
 *   slot_mapping int32 [num_tokens]; a negative slot (graph padding) skips
 *                the token.  Precondition: non-negative slots are distinct
 *                and < num_blocks*block_size (larger ones are skipped).
 *   k_cache, v_cache  the shared cache (layout above), updated in place.
 *   workspace    device scratch of at least yoco_kv_append_workspace_size()
 *                bytes (bf16 only; may be NULL when that size is 0).
 *
 * bf16 arithmetic: rms_weight multiplies either the weights (many tokens:
 * folded once into the workspace) or the activations (num_tokens <= 64 and
 * hidden a multiple of 256: the workspace is not touched); that product is
 * rounded to bf16 once.  Products accumulate in fp32 on the matrix cores,
 * the RMS scale is applied in fp32 and the result is rounded to bf16
 * (nearest-even).  fp32: plain fp32 throughout.
 *
 * Supported: hidden a positive multiple of 64; head_dim in {64, 128, 256};
 * block_size a power of two in [1, 256].
 * Errors: YOCO_ERR_INVALID_ARGUMENT, YOCO_ERR_UNSUPPORTED,
 * YOCO_ERR_WORKSPACE_TOO_SMALL.  num_tokens == 0 is a no-op.
 */
int64_t yoco_kv_append_workspace_size(int32_t dtype, int32_t hidden, int32_t num_kv_heads,
                                      int32_t head_dim);
int32_t yoco_kv_append(int32_t dtype, const void* x, int32_t num_tokens, int32_t hidden,
                       const void* rms_weight, float eps, const void* w_k, const void* w_v,
                       const int32_t* slot_mapping, void* k_cache, void* v_cache,
                       int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                       int32_t head_dim, void* workspace, int64_t workspace_bytes,
                       void* stream);

/*
 * yoco_kv_scatter -- write given K^/V^ rows into their cache slots, and
 * yoco_kv_append_fp8 -- the shared projection into an 8-bit cache.
 *
 * [KV] "Quantized cache changes attention inputs": a quantized cache stores
 * fewer bytes per scalar plus scale metadata, and keys and values may need
 * their own calibration.  [YOCO] section 18.2: quantize the shared K/V once
 * and let every cross layer reuse it.  Into a YOCO_DTYPE_FP8_E4M3 cache each
 * (token, KV head) row x of head_dim values is stored as
 *     s = max|x| / 448,  code_i = E4M3(x_i / s)
 * (both divisions fp32, round to nearest even; a zero row gives s = 0 and
 * zero codes; a row holding inf or NaN gives NaN codes), K and V with their
 * own scales; code_i * s is the stored value.
 *
 * yoco_kv_scatter:
 *   src_dtype     YOCO_DTYPE_F32 or YOCO_DTYPE_BF16: type of k_rows, v_rows.
 *   k_rows, v_rows  [num_tokens][num_kv_heads][head_dim].
 *   slot_mapping  int32 [num_tokens]; negative (or >= num_blocks*block_size)
 *                 slots are skipped.
 *   cache_dtype   src_dtype (rows copied bit for bit) or
 *                 YOCO_DTYPE_FP8_E4M3 (quantized as above).
 *   k_scale, v_scale  fp32 [num_blocks][num_kv_heads][block_size]: required
 *                 for, and only for, the FP8 cache.
 *   Supported head_dim {64, 128, 256}; block_size a power of two <= 256.
 *
 * yoco_kv_append_fp8: yoco_kv_append with the cache in FP8 E4M3: the fp32
 * projection of each token (before any bf16 rounding) is quantized.  `dtype`
 * is the type of x, rms_weight, w_k and w_v.  The workspace needs at least
 * yoco_kv_append_fp8_workspace_size() bytes: the folded weights of the bf16
 * GEMM, plus the projected fp32 rows [T][2*Hkv*D] where the projection does
 * not quantize in place (fp32 inputs, or at most 64 tokens), so it grows with
 * num_tokens only there.  Workspace and caches need 16-byte alignment, scales
 * 4-byte.
 *
 * Errors: YOCO_ERR_INVALID_ARGUMENT, YOCO_ERR_UNSUPPORTED,
 * YOCO_ERR_WORKSPACE_TOO_SMALL.  num_tokens == 0 is a no-op.
 */
int32_t yoco_kv_scatter(int32_t src_dtype, const void* k_rows, const void* v_rows, int32_t num_tokens,
                        const int32_t* slot_mapping, int32_t cache_dtype, void* k_cache, void* v_cache,
                        float* k_scale, float* v_scale, int32_t num_blocks, int32_t num_kv_heads,
                        int32_t block_size, int32_t head_dim, void* stream);
int64_t yoco_kv_append_fp8_workspace_size(int32_t dtype, int32_t num_tokens, int32_t hidden,
                                          int32_t num_kv_heads, int32_t head_dim);
int32_t yoco_kv_append_fp8(int32_t dtype, const void* x, int32_t num_tokens, int32_t hidden,
                           const void* rms_weight, float eps, const void* w_k, const void* w_v,
                           const int32_t* slot_mapping, void* k_cache, void* v_cache, float* k_scale,
                           float* v_scale, int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                           int32_t head_dim, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * yoco_cross_attn -- one cross layer's attention over the shared cache.
 *
 * [KV] "Cache contents": at decode the current query attends to every cached
 * key and value, softmax(q_t K_{<=t}^T / sqrt(d_h)) V_{<=t}.  [YOCO] sections
 * 10.4 and 13.2: each cross layer has its own query for the current position
 * only (query length 1) and reads the same K^/V^ as every other layer, over
 * the request's whole context (KV length t).  [KV] "Contiguous allocation
 * wastes capacity": every logical block is resolved through the block table.
 *
 * For request r with n = seq_lens[r] and query head h (KV head
 * g = h / (num_q_heads / num_kv_heads)):
 *     out[r][h] = sum_j softmax_j(scale * q[r][h] . K^[r][j][g]) V^[r][j][g],
 *     j = 0 .. n-1 (the current token's own K^/V^ included).
 * n == 0 gives a zero row.  A NaN in a context row gives NaN outputs.
 *
 *   dtype        type of q and the cache.
 *   q            [num_seqs][num_q_heads][head_dim].
 *   k_cache, v_cache  the shared cache (layout above), read only.
 *   block_table  int32 [num_seqs][max_blocks_per_seq].  Precondition:
 *                entries used by a context lie in [0, num_blocks).  An entry
 *                outside that range is never dereferenced and its tokens are
 *                left out of the softmax (a context whose every entry is out
 *                of range gives a zero row).
 *   seq_lens     int32 [num_seqs]; values are clamped to
 *                [0, min(max_seq_len, max_blocks_per_seq*block_size)].
 *   max_seq_len  an upper bound of seq_lens; sizes the split into partitions.
 *   scale        softmax scale; the pages' value is 1/sqrt(head_dim).
 *   partition_tokens  split-KV partition size P: a positive multiple of
 *                64 spanning at most 511 blocks and at most 16384 tokens
 *                (YOCO_ERR_UNSUPPORTED beyond); a context of n tokens is
 *                split into ceil(n/P) partitions of P tokens (the last one
 *                shorter).  0 lets the library pick P from the shape and the
 *                kernel that runs; with at most 2048 requests it also cuts
 *                the last T tokens of every context into pieces of Ps = P/4
 *                tokens (rounded down to a multiple of 64, at least 256;
 *                only when that is less than P).
 *                yoco_cross_attn_partition_split returns the plan.  The
 *                shorter pieces come after all full partitions in the
 *                schedule, so the work ends on short items.
 *   flags        YOCO_FLAG_REVERSE_ORDER or 0.
 *   out          fp32 [num_seqs][num_q_heads][head_dim].
 *   workspace    device scratch of at least yoco_cross_attn_workspace_size()
 *                bytes for the same arguments: the work-queue counters
 *                (YOCO_CROSS_ATTN_QUEUE_BYTES, zero before the first call
 *                with this workspace, left zero by every call), then the
 *                partitions' partial results, merged by a second kernel on
 *                the same stream.  Calls that may run concurrently (other
 *                streams) need separate workspaces.
 *
 * Schedule: with num_seqs <= 2048 the attention kernel keeps as many
 * workgroups as fit on the GPU at once, and each takes (request, KV head,
 * partition) work items from device-side counters until none is left;
 * partitions past the end of a context are never scheduled.  With more
 * requests every work item gets a workgroup of its own.
 *
 * Supported: head_dim in {64, 128, 256}; num_q_heads / num_kv_heads in
 * {1, 2, 4, 8}; block_size a power of two in [1, 256]; at most 65535
 * partitions per request.  The two sizing helpers return -1 for invalid
 * arguments.
 * Errors: YOCO_ERR_INVALID_ARGUMENT, YOCO_ERR_UNSUPPORTED,
 * YOCO_ERR_WORKSPACE_TOO_SMALL, YOCO_ERR_HIP.  num_seqs == 0 is a no-op.
 * Results are deterministic: the same inputs give the same bits, with or
 * without YOCO_FLAG_REVERSE_ORDER.
 */
/* P of the vector-ALU kernel's plan for these sizes (partition_tokens itself
 * when positive); yoco_cross_attn_partition_split gives either kernel's whole
 * plan. */
int32_t yoco_cross_attn_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_seq_len, int32_t block_size,
                                         int32_t partition_tokens);
/* The split of every context into partitions that yoco_cross_attn
 * (max_query_len 1, window 0) or yoco_cross_attn_varlen makes for these
 * arguments (an FP8 cache's scale arrays taken as 16-byte aligned): writes
 * split[0] = P, split[1] = Ps, split[2] = T (host array of three) and returns
 * the most partitions any query's key range gets (-1 for invalid arguments).
 * A key range of m tokens has big = m > T ? (m - T) / P : 0 partitions of P
 * tokens, then the rest, m - big * P tokens, in pieces of Ps tokens (an
 * empty range has one empty piece).  An explicit partition_tokens, or more
 * than 2048 requests, give Ps = P and T = 0.  (The workspace helpers size for
 * either kernel and do not take the cache type.) */
int32_t yoco_cross_attn_partition_split(int32_t dtype, int32_t num_seqs, int32_t max_query_len,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                        int32_t window, int32_t block_size, int32_t partition_tokens,
                                        uint32_t flags, int32_t* split);
/* The attention kernel that yoco_cross_attn (max_query_len 1, window 0) or
 * yoco_cross_attn_varlen runs for these arguments (an FP8 cache's scale
 * arrays taken as 16-byte aligned): 1 the matrix-core kernel, 0 the
 * vector-ALU kernel, -1 for invalid arguments.  Host only; for profiling and
 * reports (the results agree within the attention tolerance either way). */
int32_t yoco_cross_attn_kernel(int32_t dtype, int32_t num_seqs, int32_t max_query_len, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_seq_len, int32_t window, int32_t block_size,
                               int32_t partition_tokens, uint32_t flags);
int64_t yoco_cross_attn_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_seq_len, int32_t block_size,
                                       int32_t partition_tokens);
int32_t yoco_cross_attn(int32_t dtype, const void* q, int32_t num_seqs, int32_t num_q_heads,
                        const void* k_cache, const void* v_cache, int32_t num_blocks,
                        int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                        const int32_t* block_table, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, int32_t max_seq_len, float scale,
                        int32_t partition_tokens, uint32_t flags, float* out,
                        void* workspace, int64_t workspace_bytes, void* stream);

/*
 * yoco_cross_attn_noalloc -- yoco_cross_attn for callers that cannot allocate.
 *
 * For code that may not call hipMalloc (inside HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same computation,
 * arguments and results as yoco_cross_attn, but the workspace is a static
 * device array of YOCO_CROSS_ATTN_NOALLOC_SCRATCH_BYTES bytes inside the
 * library, one per GPU the library runs on, held until the process ends.
 * The call allocates nothing.  Its first call on a device looks up that
 * device's array and clears its work-queue counters with a small kernel on
 * `stream`; every call leaves them zero.
 *
 * All calls on one GPU share that GPU's array: calls that may overlap on one
 * GPU (different streams, or host threads without ordering) race and must
 * not be issued; use yoco_cross_attn with separate workspaces for those.
 *
 * Errors: as yoco_cross_attn; YOCO_ERR_WORKSPACE_TOO_SMALL when the call
 * needs more than YOCO_CROSS_ATTN_NOALLOC_SCRATCH_BYTES of workspace
 * (yoco_cross_attn_workspace_size() for the same arguments); YOCO_ERR_HIP
 * when the array's device address cannot be looked up.
 */
#define YOCO_CROSS_ATTN_NOALLOC_SCRATCH_BYTES (32LL * 1024 * 1024)
int32_t yoco_cross_attn_noalloc(int32_t dtype, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                const void* k_cache, const void* v_cache, int32_t num_blocks,
                                int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                int32_t partition_tokens, uint32_t flags, float* out, void* stream);

/*
 * yoco_gather_logits -- the rows of the logits positions, and the
 * cross-decoder's query offsets rebuilt from them.
 *
 * [vLLM] "Implementation in vLLM": the cross-decoder's batch is the rows at
 * the logits positions (several per request under speculative decoding), and
 * its attention metadata is rebuilt from them: each position is assigned to
 * the request whose scheduled rows hold it, the positions of each request are
 * counted, and the counts are summed into a new query_start_loc (the page's
 * example: positions [14,18,19,27] with query_start_loc [0,15,20,28] give
 * [0,1,3,4]).  Here that runs on the device without a host synchronisation.
 *
 *   hidden, num_tokens, row_bytes   as in yoco_gather_last.
 *   logits_indices  int32 [num_indices]: rows to take.  Precondition (as the
 *                   page's builder assumes): non-decreasing, so each
 *                   request's rows are consecutive in out_rows.
 *   query_start_loc int32 [num_reqs + 1] of the scheduled batch
 *                   (non-decreasing).
 *   out_rows        [num_indices][row_bytes]: out_rows[i] =
 *                   hidden[logits_indices[i]], or zero bytes when the index
 *                   lies outside [0, num_tokens).
 *   out_query_start_loc  int32 [num_reqs + 1]: 0, then the running count of
 *                   indices that lie in each request's row range; an index in
 *                   no request's range is not counted.
 *   out_max_query_len    optional int32 [1] (may be NULL): the largest count.
 *
 * Errors: YOCO_ERR_INVALID_ARGUMENT as in yoco_gather_last;
 * YOCO_ERR_UNSUPPORTED for num_reqs > 8192.  num_reqs == 0 and
 * num_indices == 0 write only what is left to write (offsets of zeros).
 */
int32_t yoco_gather_logits(const void* hidden, int64_t num_tokens, int64_t row_bytes,
                           const int32_t* logits_indices, int32_t num_indices,
                           const int32_t* query_start_loc, int32_t num_reqs, void* out_rows,
                           int32_t* out_query_start_loc, int32_t* out_max_query_len, void* stream);

/*
 * yoco_cross_attn_varlen -- one cross layer with any number of query rows per
 * request and an optional sliding window.
 *
 * [vLLM] "Implementation in vLLM": the rebuilt cross-decoder metadata keeps
 * seq_lens and is causal, so request r with n = seq_lens[r] and
 * ql = query_start_loc[r+1] - query_start_loc[r] query rows has its i-th row
 * at logical position p = n - ql + i, which attends to positions j <= p.
 * [Gemma]: a sliding-window cross layer reads only the last `window`
 * positions, p - window < j <= p.  Output row query_start_loc[r] + i:
 *     out[row][h] = sum_j softmax_j(scale * q[row][h] . K^[r][j][g]) V^[r][j][g]
 * over those j (g = h / (num_q_heads / num_kv_heads)); a row with no
 * position (p < 0, or n == 0) gives zeros.
 *
 *   dtype, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale,
 *   partition_tokens, flags, workspace: as in yoco_cross_attn, except that
 *   the partitions split the longest range a request's rows read,
 *   min(max_seq_len, window + max_query_len - 1) with a window (max_seq_len
 *   without), and the workspace size comes from
 *   yoco_cross_attn_varlen_workspace_size().
 *   q, out          [num_rows][num_q_heads][head_dim] (q in the cache dtype,
 *                   out fp32).
 *   query_start_loc int32 [num_seqs + 1], non-decreasing, values within
 *                   [0, num_rows]; NULL means one row per request (row r,
 *                   num_rows == num_seqs, max_query_len == 1), which runs
 *                   the decode kernel of yoco_cross_attn.
 *   max_query_len   an upper bound of the rows per request; a request's rows
 *                   beyond it are not written.
 *   window          0 for the whole context, else the window in tokens.
 *   dtype           cache dtype; with YOCO_DTYPE_FP8_E4M3 the caches hold
 *                   codes, q is bf16, and k_scale, v_scale (fp32
 *                   [num_blocks][num_kv_heads][block_size]) give each row's
 *                   scale: the attention reads code * scale, dequantized in
 *                   the kernel.  k_scale, v_scale must be NULL otherwise.
 *
 * With query_start_loc: num_seqs <= 2048 (YOCO_ERR_UNSUPPORTED beyond); a
 * work item streams its K^/V^ rows once for several query vectors (rows x
 * heads of one KV group): up to 16 on the matrix-core kernel, which runs an
 * FP8 cache, bf16 with several rows per request and bf16 at head_dim 256
 * (when that kernel's partitions hold at least 512 tokens) when
 * block_size >= 16 (and the scales are 16-byte aligned), up to 8 on the
 * vector kernel otherwise or with YOCO_FLAG_VECTOR_KERNEL.  A NaN in a row that some of a request's rows read
 * may give NaN in all of that request's rows.  Errors as in yoco_cross_attn.
 */
int64_t yoco_cross_attn_varlen_workspace_size(int32_t num_rows, int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                              int32_t max_query_len, int32_t window, int32_t block_size,
                                              int32_t partition_tokens);
int32_t yoco_cross_attn_varlen(int32_t dtype, const void* q, int32_t num_rows,
                               const int32_t* query_start_loc, int32_t num_seqs, int32_t max_query_len,
                               int32_t num_q_heads, const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale, int32_t num_blocks,
                               int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                               const int32_t* block_table, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t max_seq_len, int32_t window, float scale,
                               int32_t partition_tokens, uint32_t flags, float* out, void* workspace,
                               int64_t workspace_bytes, void* stream);

/*
 * yoco_gated_retention -- the self-decoder's gated retention over a batch of
 * requests (prefill chunks and decode tokens alike), with per-request states.
 *
 * [YOCO] sections 4.1-4.2: gated retention is a linear recurrence with an
 * input-dependent forget gate over a fixed-size state per head; the current
 * token's k^T v is written in and the query reads from the state; prefill
 * uses the chunkwise form, decode the recurrent one.  The page's formulas did
 * not survive; this call computes, per request and head, over the request's
 * rows in order:
 *     S_t = gamma_t * S_{t-1} + k_t^T v_t        (outer product, [D][D])
 *     o_t = q_t S_t                              (the current token included)
 * starting from the request's state slot, and writes the final S_t back to
 * the slot.  No scale or normalisation is applied.
 *
 *   dtype          YOCO_DTYPE_BF16 (q, k, v); YOCO_DTYPE_F32 returns
 *                  YOCO_ERR_UNSUPPORTED.
 *   q, k, v        [num_tokens][num_heads][head_dim], token-major, 16-byte
 *                  aligned.
 *   gamma          fp32 [num_tokens][num_heads], the gate of each token and
 *                  head, in [0, 1].  log2 gamma is clamped at -64 (a zero gate
 *                  weighs 2^-64) on the chunkwise path.
 *   head_dim       64 or 128 (key and value head_dim alike; else
 *                  YOCO_ERR_UNSUPPORTED).
 *   cu_seqlens     int32 [num_reqs + 1]: request r owns rows
 *                  cu_seqlens[r] .. cu_seqlens[r+1]-1 (clamped to
 *                  [0, num_tokens]; a request with no rows leaves its slot
 *                  untouched).  Precondition: non-decreasing (with
 *                  overlapping requests the segmented schedule computes
 *                  nothing).
 *   max_seqlen     an upper bound on any request's rows, or 0 if unknown.  It
 *                  only chooses the schedule: 1 runs the recurrent form (one
 *                  workgroup per request and head streaming its state), up to
 *                  2048 one chunkwise run per request, above (or 0) splits
 *                  long requests into 2048-row segments computed in parallel
 *                  (needs a workspace).  A request longer than max_seqlen is
 *                  still computed in full.
 *   state          fp32 [num_slots][num_heads][head_dim][head_dim] (key row,
 *                  value column), 16-byte aligned, read and updated in place.
 *   state_indices  int32 [num_reqs]: request r's slot.  A slot outside
 *                  [0, num_slots) starts from zeros and is not stored.
 *                  Requests with rows must name distinct slots (they run
 *                  concurrently).
 *   out            fp32 [num_tokens][num_heads][head_dim]: o_t of every row
 *                  owned by a request (other rows are not written).
 *   workspace      device scratch of yoco_gated_retention_workspace_size()
 *                  bytes, 16-byte aligned (may be NULL when that is 0); its
 *                  contents need no initialisation.  Calls sharing a workspace
 *                  must be ordered on one stream.
 *
 * The chunkwise form runs in 32-token chunks on the matrix cores: bf16 q, k,
 * v exact, fp32 operands (state, decayed scores, gated keys) as two bf16
 * parts, fp32 sums; the recurrent form is fp32 throughout.  Errors:
 * YOCO_ERR_INVALID_ARGUMENT (null pointers, negative counts, misalignment),
 * YOCO_ERR_UNSUPPORTED, YOCO_ERR_WORKSPACE_TOO_SMALL, YOCO_ERR_HIP.
 * num_reqs == 0 or num_tokens == 0 is a no-op.
 */
int64_t yoco_gated_retention_workspace_size(int32_t num_tokens, int32_t num_reqs, int32_t num_heads,
                                            int32_t head_dim, int32_t max_seqlen);
int32_t yoco_gated_retention(int32_t dtype, const void* q, const void* k, const void* v, const float* gamma,
                             int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                             const int32_t* cu_seqlens, int32_t num_reqs, int32_t max_seqlen, float* state,
                             int32_t num_slots, const int32_t* state_indices, float* out, void* workspace,
                             int64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* YOCO_H_ */

// yoco_cross_attn: one YOCO cross layer's attention over the shared paged cache.
//
// What is computed ("KV cache memory systems", section "Cache contents";
// "YOCO_论文与推理数据流详解" §10.4 and §13.2): every request has one query per
// query head, and it attends to the request's whole context of K^/V^ rows in
// the one cache that all cross layers share; each logical block of the
// context is found through the block table ("KV cache memory systems",
// section "Contiguous allocation wastes capacity").
//
// How (gfx950):
//   * Split-KV.  A workgroup of four wavefronts owns one work item =
//     (request, KV head, partition of `partition_tokens` context tokens), so a
//     long context still spreads over every compute unit.  The partition's
//     block-table slice is staged in LDS once; the four wavefronts take every
//     fourth iteration of the partition and combine their softmax states in
//     LDS at the end.
//   * When a request has more than one partition, each workgroup writes an
//     unnormalised partial (acc, running max m, running sum l) to the
//     workspace and a second, small kernel merges them with log-sum-exp
//     weights in partition order (deterministic).  A request that fits one
//     partition is finished by the first kernel.  The kernel boundary makes
//     the partials visible; making them visible from inside the first kernel
//     would need an agent-scope release (an L2 write-back) per workgroup,
//     and those serialise per XCD.
//   * Each K^/V^ row is read once and used for all G query heads of its KV
//     group (GQA); the G queries are staged in LDS.
//   * A row of head_dim elements is split into 16-byte chunks; LPR lanes cover
//     one row with CPL chunks each, so one wavefront load instruction reads
//     64/LPR rows, coalesced within each cache block.  The next iteration's
//     rows are loaded while the current ones are used (two register sets).
//   * q.k uses v_dot2_f32_bf16 (two bf16 products per instruction, fp32
//     accumulation) and a DPP all-reduce over the LPR lanes of a row.
//   * Online softmax in base 2 with a lazy maximum: the running max of a row
//     group is raised only when a score exceeds it by more than 2^8, so the
//     accumulators are rescaled rarely; sums stay within 256x the true terms.
//   * p.v in fp32 FMA; bf16 values widen with one shift or mask.
//   * The 64/LPR row groups of a wavefront merge by a reduce-scatter over the
//     lane's row bits (lane-half swaps, DPP, swizzle): each accumulator value
//     is rescaled and added by one lane, which ends with head_dim/64 columns.
//
// yoco_cross_attn_varlen generalises the query side ("You Only Cache Once, in
// vLLM", section "Implementation in vLLM": the cross-decoder metadata keeps
// seq_lens and marks attention causal, so a request with q logits rows has
// queries at its last q positions; Gemma 3n's sliding-window cross layers read
// a shared sliding-window cache, same page, section "Gemma 3n"):
//   * a window of W tokens restricts the query at position p to keys
//     p-W < j <= p.  With one query per request this only moves the start of
//     the range the partitions cover, so the decode kernel is unchanged.
//   * several query rows per request: a work item carries QPI consecutive
//     query rows of one request (QPI*G <= 8 "virtual heads" share every K^/V^
//     row), and each row masks the keys outside its own causal window.

#include <cmath>
#include <map>
#include <mutex>
#include <utility>

#include "cross_attn_kernels.h"

namespace yoco_attn {

// Workgroups of one kernel instance resident on the current device at once
// (compute units x workgroups per compute unit), cached per device and kernel.
int resident_workgroups(const void* kernel, int per_cu_query(int*)) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  if (per_cu_query(&per_cu) != 0 || per_cu <= 0) return 0;
  cache[key] = cus * per_cu;
  return cus * per_cu;
}

}  // namespace yoco_attn

namespace {

using namespace yoco_attn;

// ---- host side ---------------------------------------------------------------

constexpr int kMaxParts = 65535;

// Largest partition whose block-table slice fits the LDS staging array.
int32_t max_partition(int32_t block_size) {
  const int64_t cap = static_cast<int64_t>(kMaxSliceBlocks - 1) * block_size / 64 * 64;
  return static_cast<int32_t>(cap < 16384 ? cap : 16384);
}

// `fp8_matrix`: the call runs the matrix-core kernel over an 8-bit cache,
// whose items are short in time for their tokens (half the bytes), so it
// wants at least about 2048 items when every context is full length; the
// vector kernel and the matrix-core kernel over a bf16 cache at least about
// 1024.  Measured against a 2048-item floor for both matrix cases: bf16
// decode64 98.3 -> 97.1 us per layer, long512k with four rows 364.8 -> 357.0;
// FP8 long512k 184.7 -> 188.9 (worse), FP8 decode64 unchanged.
int32_t resolve_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                          int32_t block_size, int32_t requested, bool fp8_matrix) {
  if (requested > 0) return requested;
  const int64_t pairs = static_cast<int64_t>(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
  const int64_t len = max_seq_len > 0 ? max_seq_len : 1;
  const int64_t d = head_dim > 0 ? head_dim : 128;
  int64_t p;
  if (num_seqs <= kMaxQueueSeqs) {
    // Persistent schedule: items of about 2 MB of bf16 K^/V^ (P*D = 2^19),
    // but at least about 1024 items (2048 for fp8_matrix) when every context
    // is full length and at most 256 partitions per request, so the merge
    // stays small next to the stream.  Each item ends in a hand-over
    // (combine, write the partial, stage the next slice) during which the
    // workgroup has little in flight, so with the tail pieces below taking
    // care of the queue's end, long items pay: decode32x32k 694 us per layer
    // at P*D = 2^17, 668 at 2^18, 658 at 2^19, 670 at 2^20; mixed48 380,
    // 364, 363, 372 us.  Matrix kernel without pieces, against 2^17:
    // decode32x32k with an FP8 cache 401 -> 365 us, with four query rows
    // 763 -> 691 us.
    p = yoco::round_up((int64_t{1} << 19) / d, 64);
    const int64_t min_items = fp8_matrix ? 2048 : 1024;
    const int64_t p_items = yoco::round_up(yoco::ceil_div(len, yoco::ceil_div(min_items, pairs)), 64);
    if (p > p_items) p = p_items;
    if (p < 256) p = 256;
    const int64_t p_merge = yoco::round_up(yoco::ceil_div(len, 256), 64);
    if (p < p_merge) p = p_merge;
  } else {
    // One workgroup per item: about 2048 workgroups with partitions of 64
    // tokens or more.
    p = yoco::round_up(yoco::ceil_div(len, yoco::ceil_div(2048, pairs)), 64);
  }
  const int64_t cap = max_partition(block_size > 0 ? block_size : 1);
  if (p > cap) p = cap;
  if (p < 64) p = 64;
  return static_cast<int32_t>(p);
}

// Tail pieces, when the library picks the partition for the persistent
// schedule: the last T tokens of every context (and whatever is left over
// from the full partitions) are cut into pieces of P/4 tokens (at least 256,
// and only when that is less than P), which the schedule runs after every
// full partition.  The queue then ends on short items instead of leaving
// workgroups idle while the last ones finish a full partition (which cost
// about 3% of a layer on decode32x32k and 8% on long512k, with 2048-token
// partitions; with 512-token partitions at head_dim 256, 256-token pieces
// took decode64 from 102.0 to 98.7 us per layer, 71.8 to 68.2 with an FP8
// cache, where 128-token pieces or twice the tail were slower).  T is
// derived from the sizes alone (no device query, so the workspace helpers
// give the same plan): with every context full length the pieces are about
// two rounds of a nominal 512 resident workgroups, T = 256 P / (requests x
// KV heads).
constexpr int kPieceDiv = 4;
constexpr int64_t kMinPiece = 256;
constexpr int64_t kNominalSlots = 512;

Split resolve_split(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                    int32_t block_size, int32_t requested, bool fp8_matrix) {
  Split s;
  s.P = resolve_partition(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, requested, fp8_matrix);
  s.Ps = s.P;
  s.T = 0;
  // (Both kernels: since the matrix-core kernel pipelines its items, the
  // pieces pay there too -- mixed48 with an FP8 cache 214.9 -> 205.6 us per
  // layer, long512k FP8 189.0 -> 185.9 -- except with four query rows on
  // long512k, 360.8 -> 366.5.)
  if (requested > 0 || num_seqs > kMaxQueueSeqs) return s;
  const int64_t ps = s.P / kPieceDiv / 64 * 64 > kMinPiece ? s.P / kPieceDiv / 64 * 64 : kMinPiece;
  if (ps >= s.P) return s;
  const int64_t pairs = static_cast<int64_t>(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
  int64_t t = yoco::round_up(yoco::ceil_div(kNominalSlots / 2 * s.P, pairs), ps);
  const int64_t len = max_seq_len > 0 ? max_seq_len : 1;
  if (t > len) t = len;
  s.Ps = static_cast<int32_t>(ps);
  s.T = static_cast<int32_t>(t);
  return s;
}

// Whether a call runs the matrix-core kernel: where the work per byte
// outgrows the vector ALUs (an FP8 cache, or several query rows per request),
// and for a bf16 cache at head_dim 256, where the matrix kernel's four
// head_dim slices per key tile stream faster than the vector kernel's 16
// lanes per row (decode64: 110.5 -> 104.6 us per layer) -- as long as its
// items stay long: where the plan cuts the contexts into partitions shorter
// than kMinMatrixBf16Partition tokens, the vector kernel's lighter item
// hand-over wins (decode64 with a window of 512, 1024, 2048 tokens, 256-token
// partitions: 25.8 / 36.9 / 58.5 us per layer on the matrix cores, 24.5 /
// 34.3 / 55.7 on the vector ALUs; with 4096 tokens, 512-token partitions:
// 81.2 against 81.6; no window: 97.1 against 105.2).  Persistent schedule
// only.  (It reads 16-key tiles that
// lie inside one block: block_size >= 16; an FP8 cache's scale arrays must be
// 16-byte aligned.)  span is the length the partitions of the longest key
// range cover (effective_len).
constexpr int32_t kMinMatrixBf16Partition = 512;

bool matrix_kernel(int32_t dtype, int32_t num_seqs, bool several_rows, int32_t num_kv_heads, int32_t head_dim,
                   int32_t span, int32_t block_size, int32_t partition_tokens, uint32_t flags,
                   bool scales_aligned) {
  const bool f8 = dtype == YOCO_DTYPE_FP8_E4M3;
  if ((flags & YOCO_FLAG_VECTOR_KERNEL) != 0 || num_seqs > kMaxQueueSeqs || block_size < 16) return false;
  if (f8) return scales_aligned;
  if (dtype != YOCO_DTYPE_BF16) return false;
  if (several_rows) return true;
  return head_dim == 256 && resolve_partition(num_seqs, num_kv_heads, head_dim, span, block_size, partition_tokens,
                                              false) >= kMinMatrixBf16Partition;
}

// Partition slots a workspace needs for calls of these sizes with any cache
// type and flags: the larger of the two plans, the vector kernel's (which the
// matrix-core kernel shares over a bf16 cache) and the matrix-core kernel's
// over an 8-bit cache.
int32_t workspace_parts(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t span, int32_t block_size,
                        int32_t requested);

// Most partitions of any key range of at most len tokens (the workspace's
// partition slots).  Over ranges with the same number b of full partitions
// the count grows with the length, and the longest such range has b plus
// ceil((T + P - 1) / Ps) pieces; so the maximum is at len itself or at the
// longest range with one full partition fewer.
int32_t max_parts(const Split& s, int32_t len) {
  const int32_t m = len > 0 ? len : 0;
  int32_t best = s.parts(m);
  const int32_t nb = s.big(m);
  if (nb >= 1) {
    const int64_t m2 = static_cast<int64_t>(s.T) + static_cast<int64_t>(nb) * s.P - 1;
    const int32_t alt = s.parts(static_cast<int32_t>(m2));
    if (alt > best) best = alt;
  }
  return best;
}

int32_t workspace_parts(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t span, int32_t block_size,
                        int32_t requested) {
  const int32_t v = max_parts(resolve_split(num_seqs, num_kv_heads, head_dim, span, block_size, requested, false), span);
  if (num_seqs > kMaxQueueSeqs || block_size < 16) return v;        // no matrix-core kernel for these sizes
  const int32_t m = max_parts(resolve_split(num_seqs, num_kv_heads, head_dim, span, block_size, requested, true), span);
  return v > m ? v : m;
}

// Workspace: [work-queue counters, kQueueHeaderBytes][acc fp32 num_seqs*Hq*num_parts*D | pad to 256]
// [ml fp32 num_seqs*Hq*num_parts*2]; the partials only when there is more than one partition.
struct WorkspaceLayout {
  int64_t acc_offset = 0;
  int64_t ml_offset = 0;
  int64_t total = 0;
};

WorkspaceLayout workspace_layout(int32_t num_rows, int32_t num_q_heads, int32_t head_dim, int32_t num_parts) {
  WorkspaceLayout w;
  w.total = kQueueHeaderBytes;
  if (num_parts <= 1) return w;
  const int64_t slots = static_cast<int64_t>(num_rows) * num_q_heads * num_parts;
  w.acc_offset = kQueueHeaderBytes;
  w.ml_offset = yoco::round_up(w.acc_offset + slots * head_dim * 4, 256);
  w.total = w.ml_offset + slots * 2 * 4;
  return w;
}

bool supported_dim(int d) { return d == 64 || d == 128 || d == 256; }

// Length the partitions of the longest context cover: with a window, a
// request's queries see at most window + max_query_len - 1 positions.
int32_t effective_len(int32_t max_seq_len, int32_t max_qlen, int32_t window) {
  if (window <= 0) return max_seq_len;
  const int64_t span = static_cast<int64_t>(window) + (max_qlen > 1 ? max_qlen : 1) - 1;
  return static_cast<int32_t>(span < max_seq_len ? span : max_seq_len);
}

struct AttnCall {
  int32_t dtype;
  const void* q;
  int32_t num_rows;
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t max_qlen;
  int32_t num_q_heads;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  const int32_t* block_table;
  int32_t max_blocks_per_seq;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t window;
  float scale;
  int32_t partition_tokens;
  uint32_t flags;
  float* out;
  void* workspace;
  int64_t workspace_bytes;
  void* stream;
};

int32_t run_cross_attn(const AttnCall& c, const char* who) {
  using namespace yoco;
  if (c.dtype != YOCO_DTYPE_F32 && c.dtype != YOCO_DTYPE_BF16 && c.dtype != YOCO_DTYPE_FP8_E4M3)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", who, c.dtype);
  if (c.num_seqs < 0 || c.num_rows < 0 || c.num_q_heads <= 0 || c.num_kv_heads <= 0 || c.num_blocks <= 0 ||
      c.max_blocks_per_seq <= 0 || c.max_seq_len < 0 || c.partition_tokens < 0 || c.workspace_bytes < 0 ||
      c.window < 0 || c.max_qlen < 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: negative or zero size argument", who);
  if (c.qsl == nullptr && (c.num_rows != c.num_seqs || c.max_qlen != 1))
    return fail(YOCO_ERR_INVALID_ARGUMENT,
                "%s: without query_start_loc there is one query row per request (num_rows %d, num_seqs %d, "
                "max_query_len %d)", who, c.num_rows, c.num_seqs, c.max_qlen);
  if (c.num_q_heads % c.num_kv_heads != 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who,
                c.num_q_heads, c.num_kv_heads);
  if ((c.flags & ~(YOCO_FLAG_REVERSE_ORDER | YOCO_FLAG_VECTOR_KERNEL)) != 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: unknown flags", who);
  if (!std::isfinite(c.scale)) return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: scale is not finite", who);
  if (c.partition_tokens % 64 != 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: partition_tokens %d is not a multiple of 64", who,
                c.partition_tokens);
  const bool f8 = c.dtype == YOCO_DTYPE_FP8_E4M3;
  if (f8 != (c.k_scale != nullptr) || f8 != (c.v_scale != nullptr))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: cache scales are required for, and only for, an FP8 cache", who);
  const int group = c.num_q_heads / c.num_kv_heads;
  if (!supported_dim(c.head_dim))
    return fail(YOCO_ERR_UNSUPPORTED, "%s: head_dim %d not in {64,128,256}", who, c.head_dim);
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: %d query heads per KV head not in {1,2,4,8}", who, group);
  if (!is_pow2(c.block_size) || c.block_size > 256)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: block_size %d is not a power of two <= 256", who, c.block_size);
  if (c.partition_tokens > max_partition(c.block_size))
    return fail(YOCO_ERR_UNSUPPORTED, "%s: partition_tokens %d exceeds %d for block_size %d", who,
                c.partition_tokens, max_partition(c.block_size), c.block_size);
  if (c.qsl != nullptr && c.num_seqs > kMaxQueueSeqs)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: %d requests with query_start_loc exceed %d", who, c.num_seqs,
                kMaxQueueSeqs);
  if (c.num_seqs == 0 || c.num_rows == 0 || c.max_qlen == 0) return YOCO_OK;
  if (c.q == nullptr || c.k_cache == nullptr || c.v_cache == nullptr || c.block_table == nullptr ||
      c.seq_lens == nullptr || c.out == nullptr)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: null pointer", who);
  if (!aligned16(c.q) || !aligned16(c.k_cache) || !aligned16(c.v_cache) || !aligned16(c.out))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: q, caches and out must be 16-byte aligned", who);

  const int32_t span = effective_len(c.max_seq_len, c.max_qlen, c.window);
  const bool mfma = matrix_kernel(c.dtype, c.num_seqs, c.qsl != nullptr && c.max_qlen > 1, c.num_kv_heads,
                                  c.head_dim, span, c.block_size, c.partition_tokens, c.flags,
                                  aligned16(c.k_scale) && aligned16(c.v_scale));
  const Split split = resolve_split(c.num_seqs, c.num_kv_heads, c.head_dim, span, c.block_size,
                                    c.partition_tokens, mfma && c.dtype == YOCO_DTYPE_FP8_E4M3);
  const int32_t nparts = max_parts(split, span);
  if (nparts > kMaxParts)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: %d partitions per request exceed %d", who, nparts, kMaxParts);
  const int rows_wide = (mfma ? 16 : 8) / group;
  const int qpi = c.qsl == nullptr ? 0 : (c.max_qlen > 1 ? rows_wide : 1);
  const int64_t groups = qpi == 0 ? 1 : yoco::ceil_div(c.max_qlen, qpi);
  const int64_t items = static_cast<int64_t>(c.num_seqs) * c.num_kv_heads * groups * nparts;
  if (items > 0x7fffffffLL)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: %lld work items is too many", who, (long long)items);
  const WorkspaceLayout ws = workspace_layout(c.num_rows, c.num_q_heads, c.head_dim, nparts);
  if (c.workspace_bytes < ws.total)
    return fail(YOCO_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %lld bytes, need %lld", who,
                (long long)c.workspace_bytes, (long long)ws.total);
  if (c.workspace == nullptr || !aligned16(c.workspace))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: workspace must be a 16-byte aligned pointer", who);
  const int64_t merge_grid = static_cast<int64_t>(c.num_seqs) * c.max_qlen * c.num_q_heads;
  if (nparts > 1 && merge_grid * 8 > 0xffffffffLL)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: merge grid of %lld workgroups is too many", who, (long long)merge_grid);

  AttnArgs a;
  a.q = c.q;
  a.k = c.k_cache;
  a.v = c.v_cache;
  a.block_table = c.block_table;
  a.seq_lens = c.seq_lens;
  a.out = c.out;
  char* wsb = static_cast<char*>(c.workspace);
  a.ws_acc = nparts > 1 ? reinterpret_cast<float*>(wsb + ws.acc_offset) : nullptr;
  a.ws_ml = nparts > 1 ? reinterpret_cast<float*>(wsb + ws.ml_offset) : nullptr;
  a.queue = c.num_seqs <= kMaxQueueSeqs ? reinterpret_cast<uint32_t*>(wsb) : nullptr;
  a.head_stride = c.block_size * c.head_dim;
  a.block_stride = static_cast<int64_t>(c.num_kv_heads) * c.block_size * c.head_dim;
  a.num_seqs = c.num_seqs;
  a.num_q_heads = c.num_q_heads;
  a.num_kv_heads = c.num_kv_heads;
  a.num_blocks = c.num_blocks;
  a.block_size = c.block_size;
  a.bs_shift = ilog2(c.block_size);
  a.max_blocks = c.max_blocks_per_seq;
  const int64_t cap = static_cast<int64_t>(c.max_blocks_per_seq) * c.block_size;
  a.len_cap = static_cast<int32_t>(cap < c.max_seq_len ? cap : c.max_seq_len);
  a.split = split;
  a.num_parts = nparts;
  a.scale_log2 = c.scale * kLog2e;
  a.flags = c.flags;
  a.qsl = c.qsl;
  a.num_rows = c.num_rows;
  a.max_qlen = c.max_qlen;
  a.window = c.window;
  a.k_scale = c.k_scale;
  a.v_scale = c.v_scale;

  hipStream_t s = static_cast<hipStream_t>(c.stream);
  if (yoco_validation_enabled()) {
    std::vector<int32_t> table, lens, qsl;
    bool skip = false;
    int32_t st = fetch_indices(c.block_table, int64_t{c.num_seqs} * c.max_blocks_per_seq, s, table, skip, who);
    if (st == YOCO_OK) st = fetch_indices(c.seq_lens, c.num_seqs, s, lens, skip, who);
    if (st == YOCO_OK && c.qsl != nullptr) st = fetch_indices(c.qsl, int64_t{c.num_seqs} + 1, s, qsl, skip, who);
    if (st != YOCO_OK) return st;
    if (!skip && yoco_validate_block_table(table.data(), c.num_seqs, c.max_blocks_per_seq, lens.data(),
                                           c.max_seq_len, c.num_blocks, c.block_size,
                                           c.qsl != nullptr ? qsl.data() : nullptr, c.num_rows,
                                           c.window) != YOCO_OK)
      return YOCO_ERR_INVALID_ARGUMENT;
  }
  clear_launch_error();
  const int launched = mfma ? (f8 ? dispatch_mfma_fp8(c.head_dim, group, qpi, a, items, s)
                                   : dispatch_mfma_bf16(c.head_dim, group, qpi, a, items, s))
                       : c.dtype == YOCO_DTYPE_BF16 ? dispatch_bf16(c.head_dim, group, qpi, a, items, s)
                       : f8                         ? dispatch_fp8(c.head_dim, group, qpi, a, items, s)
                                                    : dispatch_f32(c.head_dim, group, qpi, a, items, s);
  if (launched == 0) return fail(YOCO_ERR_UNSUPPORTED, "%s: no kernel for this shape", who);
  if (launched < 0) return fail(YOCO_ERR_HIP, "%s: occupancy query failed on the current device", who);
  if (nparts > 1) {
    // split head_dim over up to 8 workgroups when there are fewer than ~512
    // triples, keeping at least 8 float4 slices per workgroup (at most 32
    // partition groups to combine at the end)
    int split = 1;
    while (split < 8 && merge_grid * split < 512 && c.head_dim / 4 / (split * 2) >= 8) split *= 2;
    const uint32_t mgrid = static_cast<uint32_t>(merge_grid * split);
    auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3(mgrid), dim3(kThreads), 0, s, a); };
    switch (c.head_dim * 16 + split) {
      case 64 * 16 + 1: go(cross_attn_merge_kernel<64, 1>); break;
      case 64 * 16 + 2: go(cross_attn_merge_kernel<64, 2>); break;
      case 64 * 16 + 4: go(cross_attn_merge_kernel<64, 4>); break;
      case 64 * 16 + 8: go(cross_attn_merge_kernel<64, 8>); break;
      case 128 * 16 + 1: go(cross_attn_merge_kernel<128, 1>); break;
      case 128 * 16 + 2: go(cross_attn_merge_kernel<128, 2>); break;
      case 128 * 16 + 4: go(cross_attn_merge_kernel<128, 4>); break;
      case 128 * 16 + 8: go(cross_attn_merge_kernel<128, 8>); break;
      case 256 * 16 + 1: go(cross_attn_merge_kernel<256, 1>); break;
      case 256 * 16 + 2: go(cross_attn_merge_kernel<256, 2>); break;
      case 256 * 16 + 4: go(cross_attn_merge_kernel<256, 4>); break;
      default: go(cross_attn_merge_kernel<256, 8>); break;
    }
  }
  return launch_result(who);
}

}  // namespace

// ---- the entry point that allocates nothing -----------------------------------------
//
// yoco_cross_attn_noalloc runs yoco_cross_attn with the workspace in a static
// device array instead of caller memory.  The array lives in every device's
// copy of this library's code object; host code never passes its name (a
// host-side stand-in) to a kernel, only the device address looked up once per
// device with hipGetSymbolAddress.

namespace {

static __device__ __align__(256) unsigned char scratch[YOCO_CROSS_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Zero the queue counters of one device's scratch (a kernel, not a memset,
// so that a caller's graph capture records nothing it must not replay).
__global__ __launch_bounds__(256) void clear_queue_kernel(uint32_t* queue, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) queue[i] = 0u;
}

// Device address of `scratch` on the current device, looked up (and its
// queue counters cleared on `stream`) the first time a device is seen.
int32_t scratch_of_current_device(void** out, hipStream_t stream, const char* who) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return yoco::fail(YOCO_ERR_HIP, "%s: no current device (or device index >= %d)", who, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || ptr == nullptr)
      return yoco::fail(YOCO_ERR_HIP, "%s: hipGetSymbolAddress of the static scratch failed: %s", who,
                        hipGetErrorString(err));
    yoco::clear_launch_error();
    hipLaunchKernelGGL(clear_queue_kernel, dim3(1), dim3(256), 0, stream, static_cast<uint32_t*>(ptr),
                       static_cast<int>(kQueueHeaderBytes / 4));
    const int32_t st = yoco::launch_result(who);
    if (st != YOCO_OK) return st;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return YOCO_OK;
}

}  // namespace

extern "C" int32_t yoco_cross_attn_noalloc(int32_t dtype, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                           const void* k_cache, const void* v_cache, int32_t num_blocks,
                                           int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                                           const int32_t* block_table, int32_t max_blocks_per_seq,
                                           const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                           int32_t partition_tokens, uint32_t flags, float* out, void* stream) {
  const char* who = "cross_attn_noalloc";
  // the scratch the call needs, checked before anything is looked up or launched
  if (num_seqs >= 0 && num_q_heads > 0 && num_kv_heads > 0 && head_dim > 0 && max_seq_len >= 0 && block_size > 0 &&
      partition_tokens >= 0) {
    const bool mfma = matrix_kernel(dtype, num_seqs, false, num_kv_heads, head_dim, max_seq_len, block_size,
                                    partition_tokens, flags, true);
    const Split sp = resolve_split(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, partition_tokens,
                                   mfma && dtype == YOCO_DTYPE_FP8_E4M3);
    const int64_t need = workspace_layout(num_seqs, num_q_heads, head_dim, max_parts(sp, max_seq_len)).total;
    if (need > YOCO_CROSS_ATTN_NOALLOC_SCRATCH_BYTES)
      return yoco::fail(YOCO_ERR_WORKSPACE_TOO_SMALL,
                        "%s: the call needs %lld bytes of scratch, the static scratch holds %lld (use "
                        "yoco_cross_attn with a workspace)", who, (long long)need,
                        (long long)YOCO_CROSS_ATTN_NOALLOC_SCRATCH_BYTES);
  }
  void* ws = nullptr;
  if (num_seqs > 0) {
    const int32_t st = scratch_of_current_device(&ws, static_cast<hipStream_t>(stream), who);
    if (st != YOCO_OK) return st;
  }
  const AttnCall c{dtype, q, num_seqs, nullptr, num_seqs, 1, num_q_heads, k_cache, v_cache, nullptr, nullptr,
                   num_blocks, num_kv_heads, block_size, head_dim, block_table, max_blocks_per_seq, seq_lens,
                   max_seq_len, 0, scale, partition_tokens, flags, out, ws,
                   ws == nullptr ? 0 : YOCO_CROSS_ATTN_NOALLOC_SCRATCH_BYTES, stream};
  return run_cross_attn(c, who);
}

extern "C" int32_t yoco_cross_attn_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_seq_len, int32_t block_size,
                                                    int32_t partition_tokens) {
  if (partition_tokens < 0 || max_seq_len < 0 || block_size <= 0) return -1;
  return resolve_partition(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, partition_tokens, false);
}

extern "C" int32_t yoco_cross_attn_partition_split(int32_t dtype, int32_t num_seqs, int32_t max_query_len,
                                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                                   int32_t window, int32_t block_size, int32_t partition_tokens,
                                                   uint32_t flags, int32_t* split) {
  if (partition_tokens < 0 || max_seq_len < 0 || max_query_len < 0 || window < 0 || block_size <= 0 ||
      split == nullptr)
    return -1;
  const int32_t span = effective_len(max_seq_len, max_query_len, window);
  const bool mfma = matrix_kernel(dtype, num_seqs, max_query_len > 1, num_kv_heads, head_dim, span, block_size,
                                  partition_tokens, flags, true);
  const Split s = resolve_split(num_seqs, num_kv_heads, head_dim, span, block_size, partition_tokens,
                                mfma && dtype == YOCO_DTYPE_FP8_E4M3);
  split[0] = s.P;
  split[1] = s.Ps;
  split[2] = s.T;
  return max_parts(s, span);
}

extern "C" int32_t yoco_cross_attn_kernel(int32_t dtype, int32_t num_seqs, int32_t max_query_len,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                          int32_t window, int32_t block_size, int32_t partition_tokens,
                                          uint32_t flags) {
  if (partition_tokens < 0 || max_seq_len < 0 || max_query_len < 0 || window < 0 || block_size <= 0 ||
      num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0)
    return -1;
  const int32_t span = effective_len(max_seq_len, max_query_len, window);
  return matrix_kernel(dtype, num_seqs, max_query_len > 1, num_kv_heads, head_dim, span, block_size,
                       partition_tokens, flags, true)
             ? 1
             : 0;
}

extern "C" int64_t yoco_cross_attn_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t max_seq_len, int32_t block_size,
                                                  int32_t partition_tokens) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      block_size <= 0 || partition_tokens < 0)
    return -1;
  return workspace_layout(num_seqs, num_q_heads, head_dim,
                          workspace_parts(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, partition_tokens))
      .total;
}

extern "C" int64_t yoco_cross_attn_varlen_workspace_size(int32_t num_rows, int32_t num_seqs, int32_t num_q_heads,
                                                         int32_t num_kv_heads, int32_t head_dim,
                                                         int32_t max_seq_len, int32_t max_query_len,
                                                         int32_t window, int32_t block_size,
                                                         int32_t partition_tokens) {
  if (num_rows < 0 || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      max_query_len < 0 || window < 0 || block_size <= 0 || partition_tokens < 0)
    return -1;
  const int32_t span = effective_len(max_seq_len, max_query_len, window);
  return workspace_layout(num_rows, num_q_heads, head_dim,
                          workspace_parts(num_seqs, num_kv_heads, head_dim, span, block_size, partition_tokens))
      .total;
}

extern "C" int32_t yoco_cross_attn(int32_t dtype, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                   const void* k_cache, const void* v_cache, int32_t num_blocks,
                                   int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                   int32_t partition_tokens, uint32_t flags, float* out, void* workspace,
                                   int64_t workspace_bytes, void* stream) {
  const AttnCall c{dtype, q, num_seqs, nullptr, num_seqs, 1, num_q_heads, k_cache, v_cache, nullptr, nullptr,
                   num_blocks, num_kv_heads, block_size, head_dim, block_table, max_blocks_per_seq, seq_lens,
                   max_seq_len, 0, scale, partition_tokens, flags, out, workspace, workspace_bytes, stream};
  return run_cross_attn(c, "cross_attn");
}

extern "C" int32_t yoco_cross_attn_varlen(int32_t dtype, const void* q, int32_t num_rows,
                                          const int32_t* query_start_loc, int32_t num_seqs, int32_t max_query_len,
                                          int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                          const float* k_scale, const float* v_scale, int32_t num_blocks,
                                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                                          const int32_t* block_table, int32_t max_blocks_per_seq,
                                          const int32_t* seq_lens, int32_t max_seq_len, int32_t window,
                                          float scale, int32_t partition_tokens, uint32_t flags, float* out,
                                          void* workspace, int64_t workspace_bytes, void* stream) {
  const AttnCall c{dtype, q, num_rows, query_start_loc, num_seqs, max_query_len, num_q_heads, k_cache, v_cache,
                   k_scale, v_scale, num_blocks, num_kv_heads, block_size, head_dim, block_table,
                   max_blocks_per_seq, seq_lens, max_seq_len, window, scale, partition_tokens, flags, out,
                   workspace, workspace_bytes, stream};
  return run_cross_attn(c, "cross_attn_varlen");
}

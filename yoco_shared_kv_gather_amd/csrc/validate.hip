// Checks of the device-side preconditions of the library's calls, on host
// copies of the index arrays.
//
// The calls never validate index data on the device: each kernel clamps or
// skips an index that breaks a precondition, so nothing is read or written
// outside the buffers, but the affected rows' results are then unspecified.
// To find such inputs while debugging, YOCO_VALIDATE=1 in the environment (or
// yoco_set_validation(1)) makes every call copy its index arrays to the host,
// synchronise its stream, and return YOCO_ERR_INVALID_ARGUMENT with the first
// violation before launching anything.  The preconditions are those of the
// pages' metadata: every logical block of a context resolves through the
// block table to a physical page ("KV cache memory systems", section
// "Contiguous allocation wastes capacity"); query_start_loc / cu_seqlens are
// offsets of consecutive rows, slot_mapping names distinct slots, and
// logits_indices are in order ("You Only Cache Once, in vLLM", section
// "Implementation in vLLM").  The host-array checks are also exported
// (yoco_validate_*), so a caller can run them on metadata it already holds.

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "yoco_internal.h"

namespace {

// -1: not read yet; 0 / 1: off / on
std::atomic<int> g_validation{-1};

constexpr int32_t kInvalid = YOCO_ERR_INVALID_ARGUMENT;

int range_lo(int n, int ql, int window) {
  if (window <= 0) return 0;
  const int lo = n - ql - window + 1;
  return lo > 0 ? lo : 0;
}

}  // namespace

extern "C" {

void yoco_set_validation(int32_t enabled) { g_validation.store(enabled ? 1 : 0); }

int32_t yoco_validation_enabled(void) {
  int v = g_validation.load();
  if (v < 0) {
    const char* env = std::getenv("YOCO_VALIDATE");
    v = (env != nullptr && env[0] != '\0' && std::strcmp(env, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_validation.compare_exchange_strong(expected, v);
    v = g_validation.load();
  }
  return v;
}

int32_t yoco_validate_offsets(const int32_t* offsets, int32_t num_reqs, int64_t num_rows) {
  const char* who = "validate offsets";
  if (num_reqs < 0 || num_rows < 0)
    return yoco::fail(kInvalid, "%s: negative count (%d requests, %lld rows)", who, num_reqs, (long long)num_rows);
  if (num_reqs == 0) return YOCO_OK;
  if (offsets == nullptr) return yoco::fail(kInvalid, "%s: null offsets", who);
  for (int32_t r = 0; r <= num_reqs; ++r) {
    if (offsets[r] < 0 || offsets[r] > num_rows)
      return yoco::fail(kInvalid, "%s: offset %d is %d, outside [0, %lld]", who, r, offsets[r], (long long)num_rows);
    if (r > 0 && offsets[r] < offsets[r - 1])
      return yoco::fail(kInvalid, "%s: offsets decrease at request %d (%d after %d)", who, r - 1, offsets[r],
                        offsets[r - 1]);
  }
  return YOCO_OK;
}

int32_t yoco_validate_slots(const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                            int32_t block_size) {
  const char* who = "validate slot_mapping";
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0)
    return yoco::fail(kInvalid, "%s: bad sizes (%d tokens, %d blocks of %d)", who, num_tokens, num_blocks, block_size);
  if (num_tokens == 0) return YOCO_OK;
  if (slot_mapping == nullptr) return yoco::fail(kInvalid, "%s: null slot_mapping", who);
  const int64_t slots = static_cast<int64_t>(num_blocks) * block_size;
  std::vector<std::pair<int32_t, int32_t>> used;
  used.reserve(static_cast<size_t>(num_tokens));
  for (int32_t t = 0; t < num_tokens; ++t) {
    const int32_t s = slot_mapping[t];
    if (s < 0) continue;                                   // graph padding
    if (s >= slots)
      return yoco::fail(kInvalid, "%s: token %d has slot %d, past the cache's %lld slots", who, t, s, (long long)slots);
    used.emplace_back(s, t);
  }
  std::sort(used.begin(), used.end());
  for (size_t i = 1; i < used.size(); ++i)
    if (used[i].first == used[i - 1].first)
      return yoco::fail(kInvalid, "%s: tokens %d and %d share slot %d", who, used[i - 1].second, used[i].second,
                        used[i].first);
  return YOCO_OK;
}

int32_t yoco_validate_block_table(const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
                                  const int32_t* seq_lens, int32_t max_seq_len, int32_t num_blocks,
                                  int32_t block_size, const int32_t* query_start_loc, int32_t num_rows,
                                  int32_t window) {
  const char* who = "validate block_table";
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_seq_len < 0 || num_blocks <= 0 || block_size <= 0 ||
      window < 0)
    return yoco::fail(kInvalid, "%s: bad sizes (%d requests, %d table entries, %d blocks)", who, num_seqs,
                      max_blocks_per_seq, num_blocks);
  if (num_seqs == 0) return YOCO_OK;
  if (block_table == nullptr || seq_lens == nullptr) return yoco::fail(kInvalid, "%s: null table or seq_lens", who);
  if (query_start_loc != nullptr) {
    const int32_t st = yoco_validate_offsets(query_start_loc, num_seqs, num_rows);
    if (st != YOCO_OK) return st;
  }
  const int64_t row_tokens = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  for (int32_t r = 0; r < num_seqs; ++r) {
    const int32_t n = seq_lens[r];
    if (n < 0) return yoco::fail(kInvalid, "%s: seq_lens[%d] = %d is negative", who, r, n);
    if (n > max_seq_len)
      return yoco::fail(kInvalid, "%s: seq_lens[%d] = %d exceeds max_seq_len %d", who, r, n, max_seq_len);
    if (n > row_tokens)
      return yoco::fail(kInvalid, "%s: seq_lens[%d] = %d does not fit a table row of %lld tokens", who, r, n,
                        (long long)row_tokens);
    const int ql = query_start_loc == nullptr ? 1 : query_start_loc[r + 1] - query_start_loc[r];
    if (n == 0 || ql <= 0) continue;
    // the blocks the call reads: from the first position any query sees
    const int first = range_lo(n, ql, window) / block_size;
    const int last = (n - 1) / block_size;
    const int32_t* row = block_table + static_cast<int64_t>(r) * max_blocks_per_seq;
    for (int b = first; b <= last; ++b)
      if (row[b] < 0 || row[b] >= num_blocks)
        return yoco::fail(kInvalid, "%s: request %d, logical block %d maps to page %d, outside a pool of %d", who,
                          r, b, row[b], num_blocks);
  }
  return YOCO_OK;
}

int32_t yoco_validate_logits_indices(const int32_t* logits_indices, int32_t num_indices,
                                     const int32_t* query_start_loc, int32_t num_reqs, int64_t num_tokens) {
  const char* who = "validate logits_indices";
  if (num_indices < 0) return yoco::fail(kInvalid, "%s: negative count %d", who, num_indices);
  const int32_t st = yoco_validate_offsets(query_start_loc, num_reqs, num_tokens);
  if (st != YOCO_OK) return st;
  if (num_indices > 0 && logits_indices == nullptr) return yoco::fail(kInvalid, "%s: null indices", who);
  const int64_t hi = num_reqs > 0 ? query_start_loc[num_reqs] : 0;
  const int64_t lo = num_reqs > 0 ? query_start_loc[0] : 0;
  for (int32_t i = 0; i < num_indices; ++i) {
    const int32_t x = logits_indices[i];
    if (x < lo || x >= hi)
      return yoco::fail(kInvalid, "%s: index %d is %d, outside the batch's rows [%lld, %lld)", who, i, x,
                        (long long)lo, (long long)hi);
    if (i > 0 && x < logits_indices[i - 1])
      return yoco::fail(kInvalid, "%s: indices decrease at %d (%d after %d)", who, i, x, logits_indices[i - 1]);
  }
  return YOCO_OK;
}

int32_t yoco_validate_state_indices(const int32_t* state_indices, int32_t num_reqs, int32_t num_slots) {
  const char* who = "validate state_indices";
  if (num_reqs < 0 || num_slots < 0)
    return yoco::fail(kInvalid, "%s: negative count (%d requests, %d slots)", who, num_reqs, num_slots);
  if (num_reqs == 0) return YOCO_OK;
  if (state_indices == nullptr) return yoco::fail(kInvalid, "%s: null state_indices", who);
  std::vector<std::pair<int32_t, int32_t>> used;
  for (int32_t r = 0; r < num_reqs; ++r) {
    const int32_t s = state_indices[r];
    if (s < 0) continue;                                   // starts from zeros, stores nothing
    if (s >= num_slots) return yoco::fail(kInvalid, "%s: request %d has state slot %d of %d", who, r, s, num_slots);
    used.emplace_back(s, r);
  }
  std::sort(used.begin(), used.end());
  for (size_t i = 1; i < used.size(); ++i)
    if (used[i].first == used[i - 1].first)
      return yoco::fail(kInvalid, "%s: requests %d and %d share state slot %d", who, used[i - 1].second,
                        used[i].second, used[i].first);
  return YOCO_OK;
}

}  // extern "C"

namespace yoco {

int32_t fetch_indices(const int32_t* src, int64_t count, hipStream_t stream, std::vector<int32_t>& dst, bool& skip,
                      const char* who) {
  skip = false;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone) {
    skip = true;
    return YOCO_OK;
  }
  dst.assign(static_cast<size_t>(count > 0 ? count : 0), 0);
  if (count <= 0 || src == nullptr) return YOCO_OK;
  if (hipMemcpyAsync(dst.data(), src, static_cast<size_t>(count) * 4, hipMemcpyDefault, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(YOCO_ERR_HIP, "%s: copying index data to the host for validation failed", who);
  return YOCO_OK;
}

}  // namespace yoco

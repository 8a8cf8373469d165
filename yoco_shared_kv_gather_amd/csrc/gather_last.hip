// yoco_gather_last: keep each request's last scheduled token.
//
// "You Only Cache Once, in vLLM", section "Implementation in vLLM": inside
// one mixed prefill/decode step the cross-decoder processes a single token per
// request, the last one scheduled, so its batch shrinks from the scheduled
// token count to the request count.  "YOCO_论文与推理数据流详解" §7.4: only the
// last prompt position enters the cross-decoder at prefill.
//
// One workgroup per request copies the row with 16-byte loads and stores; the
// row index comes from cu_seqlens.  The copy is bitwise.
//
// yoco_gather_logits is the general form from the same section: the rows at
// the logits positions (several per request under speculative decoding) and
// the cross-decoder's query_start_loc rebuilt from them.  The page's builder
// assigns each position to its request (bucketize), counts them per request
// (bincount) and sums the counts (cumsum), reading the maximum back to the
// host; here one workgroup does all three in LDS and writes the maximum to
// device memory, so the step needs no host synchronisation.

#include "yoco_internal.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gather_last_kernel(
    const uint4* __restrict__ hidden, int64_t num_tokens, int64_t row_chunks,
    const int32_t* __restrict__ cu_seqlens, uint4* __restrict__ out,
    int32_t* __restrict__ out_index) {
  const int64_t r = blockIdx.x;
  const int32_t begin = cu_seqlens[r];
  const int32_t end = cu_seqlens[r + 1];
  const int64_t row = static_cast<int64_t>(end) - 1;
  const bool valid = end > begin && row >= 0 && row < num_tokens;
  if (out_index != nullptr && threadIdx.x == 0) out_index[r] = valid ? static_cast<int32_t>(row) : -1;
  uint4* dst = out + r * row_chunks;
  if (valid) {
    const uint4* src = hidden + row * row_chunks;
    for (int64_t c = threadIdx.x; c < row_chunks; c += kThreads) dst[c] = src[c];
  } else {
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t c = threadIdx.x; c < row_chunks; c += kThreads) dst[c] = zero;
  }
}

// out[i] = hidden[index[i]] bit for bit (zero bytes for an index outside
// [0, num_tokens)); one workgroup per selected row.
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(
    const uint4* __restrict__ hidden, int64_t num_tokens, int64_t row_chunks,
    const int32_t* __restrict__ index, uint4* __restrict__ out) {
  const int64_t i = blockIdx.x;
  const int64_t row = index[i];
  uint4* dst = out + i * row_chunks;
  if (row >= 0 && row < num_tokens) {
    const uint4* src = hidden + row * row_chunks;
    for (int64_t c = threadIdx.x; c < row_chunks; c += kThreads) dst[c] = src[c];
  } else {
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t c = threadIdx.x; c < row_chunks; c += kThreads) dst[c] = zero;
  }
}

constexpr int kMetaThreads = 1024;
constexpr int kMaxMetaReqs = 8192;

// The cross-decoder's query offsets from the logits positions, in one
// workgroup: each position finds the request r with qsl[r] <= idx < qsl[r+1]
// (binary search over the non-decreasing offsets; none if it lies outside
// every request's rows) and counts itself there with an LDS atomic; a block
// scan of the counts gives out_qsl = [0, c0, c0+c1, ...] and the largest
// count.
__global__ __launch_bounds__(kMetaThreads) void cross_metadata_kernel(
    const int32_t* __restrict__ index, int32_t num_indices, const int32_t* __restrict__ qsl, int32_t num_reqs,
    int32_t* __restrict__ out_qsl, int32_t* __restrict__ out_max) {
  __shared__ int32_t counts[kMaxMetaReqs];
  __shared__ int32_t wave_sum[kMetaThreads / 64];
  __shared__ int32_t wave_max[kMetaThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int r = tid; r < num_reqs; r += kMetaThreads) counts[r] = 0;
  __syncthreads();
  for (int i = tid; i < num_indices; i += kMetaThreads) {
    const int32_t idx = index[i];
    // largest r in [0, num_reqs) with qsl[r] <= idx, or -1
    int lo = -1, hi = num_reqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (qsl[mid] <= idx) lo = mid; else hi = mid - 1;
    }
    if (lo >= 0 && idx < qsl[lo + 1]) atomicAdd(&counts[lo], 1);
  }
  __syncthreads();
  // Thread t owns counts [t*per, (t+1)*per): local sums, a wave scan, then
  // the waves' totals.
  const int per = (num_reqs + kMetaThreads - 1) / kMetaThreads;
  const int b = min(tid * per, num_reqs);
  const int e = min(b + per, num_reqs);
  int local = 0, mx = 0;
  for (int r = b; r < e; ++r) {
    local += counts[r];
    mx = max(mx, counts[r]);
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
  if (lane == 63) wave_sum[wave] = incl;
  if (lane == 0) wave_max[wave] = mx;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wave_sum[w];
  for (int r = b; r < e; ++r) {
    run += counts[r];
    out_qsl[r + 1] = run;
  }
  if (tid == 0) {
    out_qsl[0] = 0;
    if (out_max != nullptr) {
      int m = 0;
      for (int w = 0; w < kMetaThreads / 64; ++w) m = max(m, wave_max[w]);
      *out_max = m;
    }
  }
}

}  // namespace

extern "C" int32_t yoco_gather_logits(const void* hidden, int64_t num_tokens, int64_t row_bytes,
                                      const int32_t* logits_indices, int32_t num_indices,
                                      const int32_t* query_start_loc, int32_t num_reqs, void* out_rows,
                                      int32_t* out_query_start_loc, int32_t* out_max_query_len, void* stream) {
  using namespace yoco;
  if (num_reqs < 0 || num_tokens < 0 || num_indices < 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gather_logits: negative count");
  if (num_reqs > kMaxMetaReqs)
    return fail(YOCO_ERR_UNSUPPORTED, "gather_logits: %d requests exceed %d", num_reqs, kMaxMetaReqs);
  if (query_start_loc == nullptr || out_query_start_loc == nullptr ||
      (num_indices > 0 && (logits_indices == nullptr || out_rows == nullptr)) ||
      (hidden == nullptr && num_tokens > 0 && num_indices > 0))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gather_logits: null pointer");
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gather_logits: row_bytes %lld is not a positive multiple of 16",
                static_cast<long long>(row_bytes));
  if (!aligned16(hidden) || !aligned16(out_rows))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gather_logits: hidden and out_rows must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (yoco_validation_enabled()) {
    std::vector<int32_t> idx, qsl;
    bool skip = false;
    int32_t st = fetch_indices(logits_indices, num_indices, s, idx, skip, "gather_logits");
    if (st == YOCO_OK) st = fetch_indices(query_start_loc, int64_t{num_reqs} + 1, s, qsl, skip, "gather_logits");
    if (st != YOCO_OK) return st;
    if (!skip && yoco_validate_logits_indices(idx.data(), num_indices, qsl.data(), num_reqs, num_tokens) != YOCO_OK)
      return YOCO_ERR_INVALID_ARGUMENT;
  }
  clear_launch_error();
  if (num_indices > 0)
    hipLaunchKernelGGL(gather_rows_kernel, dim3(num_indices), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(hidden), num_tokens, row_bytes / 16, logits_indices,
                       static_cast<uint4*>(out_rows));
  hipLaunchKernelGGL(cross_metadata_kernel, dim3(1), dim3(kMetaThreads), 0, s, logits_indices, num_indices,
                     query_start_loc, num_reqs, out_query_start_loc, out_max_query_len);
  return launch_result("gather_logits");
}

extern "C" int32_t yoco_gather_last(const void* hidden, int64_t num_tokens, int64_t row_bytes,
                                    const int32_t* cu_seqlens, int32_t num_reqs, void* out,
                                    int32_t* out_index, void* stream) {
  using namespace yoco;
  if (num_reqs < 0 || num_tokens < 0) return fail(YOCO_ERR_INVALID_ARGUMENT, "gather_last: negative count");
  if (num_reqs == 0) return YOCO_OK;
  if (cu_seqlens == nullptr || out == nullptr || (hidden == nullptr && num_tokens > 0))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gather_last: null pointer");
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gather_last: row_bytes %lld is not a positive multiple of 16",
                static_cast<long long>(row_bytes));
  if (!aligned16(hidden) || !aligned16(out))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gather_last: hidden and out must be 16-byte aligned");
  if (yoco_validation_enabled()) {
    std::vector<int32_t> cu;
    bool skip = false;
    const int32_t st = fetch_indices(cu_seqlens, int64_t{num_reqs} + 1, static_cast<hipStream_t>(stream), cu, skip,
                                     "gather_last");
    if (st != YOCO_OK) return st;
    if (!skip && yoco_validate_offsets(cu.data(), num_reqs, num_tokens) != YOCO_OK) return YOCO_ERR_INVALID_ARGUMENT;
  }
  clear_launch_error();
  hipLaunchKernelGGL(gather_last_kernel, dim3(num_reqs), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(hidden), num_tokens,
                     row_bytes / 16, cu_seqlens, static_cast<uint4*>(out), out_index);
  return launch_result("gather_last");
}

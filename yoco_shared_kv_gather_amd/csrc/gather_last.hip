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

}  // namespace

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
  clear_launch_error();
  hipLaunchKernelGGL(gather_last_kernel, dim3(num_reqs), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(hidden), num_tokens,
                     row_bytes / 16, cu_seqlens, static_cast<uint4*>(out), out_index);
  return launch_result("gather_last");
}

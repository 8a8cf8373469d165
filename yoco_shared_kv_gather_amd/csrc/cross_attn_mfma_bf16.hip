// yoco_cross_attn matrix-core kernels for the bf16 cache (instantiated here
// so they compile in parallel with the other element types).
#include "cross_attn_kernels.h"

namespace yoco_attn {

int dispatch_mfma_bf16(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  return dispatch_dim_mfma<kBF16>(head_dim, group, qpi, a, items, stream);
}

}  // namespace yoco_attn

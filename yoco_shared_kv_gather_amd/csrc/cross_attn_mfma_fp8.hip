// yoco_cross_attn matrix-core kernels for the fp8 cache (instantiated here
// so they compile in parallel with the other element types).
#include "cross_attn_kernels.h"

namespace yoco_attn {

int dispatch_mfma_fp8(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  return dispatch_dim_mfma<kFP8>(head_dim, group, qpi, a, items, stream);
}

}  // namespace yoco_attn

// decode_kernel instances for head_dim 128, 3-bit packed cache.
#include "decode_kernel.cuh"

namespace pkv {

const void* decode_kernel_ptr_u3_d128(int group, bool bf16, int hpi) {
  return kernel_by_dtype<128, CacheKind::U3>(group, bf16, hpi);
}

}  // namespace pkv

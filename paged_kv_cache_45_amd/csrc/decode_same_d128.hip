// decode_kernel instances for head_dim 128, bf16 / fp16 cache.
#include "decode_kernel.cuh"

namespace pkv {

const void* decode_kernel_ptr_same_d128(int group, bool bf16, int hpi) {
  return kernel_by_dtype<128, CacheKind::Same>(group, bf16, hpi);
}

}  // namespace pkv

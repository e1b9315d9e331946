// decode_kernel instances for head_dim 64, int8 cache.
#include "decode_kernel.cuh"

namespace pkv {

const void* decode_kernel_ptr_i8_d64(int group, bool bf16, int hpi) {
  return kernel_by_dtype<64, CacheKind::I8>(group, bf16, hpi);
}

}  // namespace pkv

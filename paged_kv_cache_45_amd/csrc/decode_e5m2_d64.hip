// decode_kernel instances for head_dim 64, fp8 e5m2 cache.
#include "decode_kernel.cuh"

namespace pkv {

const void* decode_kernel_ptr_e5m2_d64(int group, bool bf16, int hpi) {
  return kernel_by_dtype<64, CacheKind::E5m2>(group, bf16, hpi);
}

}  // namespace pkv

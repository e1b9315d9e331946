// decode_kernel instances for head_dim 128, fp8 e4m3fn cache.
#include "decode_kernel.cuh"

namespace pkv {

const void* decode_kernel_ptr_fp8_d128(int group, bool bf16, int hpi) {
  return kernel_by_dtype<128, CacheKind::Fp8>(group, bf16, hpi);
}

}  // namespace pkv

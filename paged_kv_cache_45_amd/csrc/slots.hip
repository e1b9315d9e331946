// Slot ids of new tokens from their request and position: the launcher's step of the append.
//
// "Write Triton Kv Cache Append Kernel", Inputs items 6 and 7 and Required reasoning process
// step 9: the paged slot id of position p of request r is block_tables[r, p / block_size] *
// block_size + p % block_size (the physical block, not the logical one); a decode token sits
// at the context length before it is incremented, which the caller passes as its position.
// Without a block table the cache is the contiguous [batch, num_kv_heads, max_seq_len,
// head_dim] one and the id is r * max_seq_len + p (block_size = max_seq_len).  Padding tokens
// (request < 0), requests >= batch and positions outside the table row or the sequence get -1,
// which the append skips.  One thread per token; no table entry outside the row is read.
#include "launch.h"

namespace pkv {

__global__ __launch_bounds__(256) void slot_kernel(SlotParams p) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= p.num_tokens) return;
  const int32_t r = p.token_request ? p.token_request[t] : (int32_t)t;
  const int32_t pos = p.token_position[t];
  int64_t slot = -1;
  if (r >= 0 && r < p.batch && pos >= 0) {
    const int64_t bs = (int64_t)1 << p.log2_bs;
    if (p.block_tables == nullptr) {
      if (pos < bs) slot = (int64_t)r * bs + pos;
    } else {
      const int64_t j = (int64_t)pos >> p.log2_bs;
      if (j < p.bt_sb) slot = (int64_t)p.block_tables[(int64_t)r * p.bt_sb + j] * bs + (pos & (bs - 1));
    }
  }
  p.slot_mapping[t] = slot;
}

hipError_t launch_slots(const SlotParams& p, hipStream_t s) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t blocks = (p.num_tokens + 255) / 256;
  hipLaunchKernelGGL(slot_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv

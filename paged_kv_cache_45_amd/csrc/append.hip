// KV append: write new K/V rows into the paged block pool through slot_mapping.
//
// "Write Triton Kv Cache Append Kernel", Required reasoning process steps 1-8:
// slot < 0 marks padding and nothing of that token is loaded; block = slot / block_size,
// offset = slot % block_size (shift and mask, block_size a power of two); K and V are
// written by the same thread group; quantised caches divide by the scale in fp32 and
// only then convert (fp8 e4m3fn, fp8 e5m2 and int8 arithmetic in fp8_quant.cuh).  The 3-bit cache follows
// "triton-3bit-kv-cache-kernel" README, sections 1A/1B (bit layout) and section 2 test 3
// (fp16 affine scale and zero).
//
// Work mapping (wave64): one (token, kv head) row per group of D/8 lanes, each lane
// owning 8 consecutive elements (one 16-byte load of K and one of V).  A 256-thread
// block covers 16 rows (D = 128) or 32 rows (D = 64).  The quantisers reduce over the
// row with DPP inside the lane group, so no barrier and no LDS are involved.
#include "append_rows.cuh"

namespace pkv {

// Each group of D/8 lanes handles R rows (token, kv head), RPB rows apart, so that the
// block covers R * RPB consecutive rows: all slot ids are loaded first, then the K/V rows of
// the valid ones, so R rows share one load latency.
template <int D, bool BF16, CacheKind KIND, int R>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int c = threadIdx.x % LPR;
  const uint32_t row0 = blockIdx.x * (uint32_t)(RPB * R) + threadIdx.x / LPR;
  const uint32_t H = (uint32_t)p.num_kv_heads;
  int64_t slot[R];
  uint32_t tok[R], head[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const uint32_t row = row0 + k * RPB;
    tok[k] = row / H;
    head[k] = row - tok[k] * H;
    slot[k] = tok[k] < (uint64_t)p.num_tokens ? p.slots[tok[k]] : -1;
  }
  bool valid[R];
  uint4 kx[R], vx[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    valid[k] = slot[k] >= 0 && slot[k] < p.capacity;   // padding: no load, no store
    if (valid[k]) {
      // the new rows are read once: streamed (measured on the mixed fp8 append: +9 %)
      kx[k] = load_stream_u4(static_cast<const uint16_t*>(p.k_new) +
                             (int64_t)tok[k] * p.k_st + (int64_t)head[k] * p.k_sh + c * 8);
      vx[k] = load_stream_u4(static_cast<const uint16_t*>(p.v_new) +
                             (int64_t)tok[k] * p.v_st + (int64_t)head[k] * p.v_sh + c * 8);
    }
  }
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (!valid[k]) continue;
    const int64_t blk = slot[k] >> p.log2_bs;
    const int64_t off = slot[k] & ((1 << p.log2_bs) - 1);
    const int64_t crow = blk * p.c_sb + off * p.c_ss + (int64_t)head[k] * p.c_sh;
    const int64_t mrow = blk * p.m_sb + off * p.m_ss + (int64_t)head[k] * p.m_sh;
    store_kv_row<LPR, BF16, KIND>(kx[k], vx[k], p.k_cache, p.v_cache, p.k_meta, p.v_meta, crow, mrow, c,
                                  p.given_scale != 0);
  }
}

// Rows per lane group: the bit copy takes 4 once the batch fills the chip several times over
// (more bytes in flight per wave); a small decode append is one latency chain either way and
// wants as many workgroups as possible.  The quantising kinds are bound by their arithmetic,
// which 4 rows per lane only serialise (measured slower), so they keep 1.
constexpr int64_t kAppendManyRows = 256 * 64;

template <int D, bool BF16, CacheKind KIND>
static hipError_t launch_append_t(const AppendParams& p, hipStream_t s) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = p.num_tokens * p.num_kv_heads;
  if (KIND == CacheKind::Same && rows >= kAppendManyRows) {
    const int64_t blocks = (rows + 4 * RPB - 1) / (4 * RPB);
    hipLaunchKernelGGL((append_kernel<D, BF16, KIND, 4>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  } else {
    const int64_t blocks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((append_kernel<D, BF16, KIND, 1>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t dispatch_kind(const AppendParams& p, CacheKind kind, hipStream_t s) {
  switch (kind) {
    case CacheKind::Same: return launch_append_t<D, BF16, CacheKind::Same>(p, s);
    case CacheKind::Fp8: return launch_append_t<D, BF16, CacheKind::Fp8>(p, s);
    case CacheKind::U3: return launch_append_t<D, BF16, CacheKind::U3>(p, s);
    case CacheKind::E5m2: return launch_append_t<D, BF16, CacheKind::E5m2>(p, s);
    case CacheKind::I8: return launch_append_t<D, BF16, CacheKind::I8>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_append(const AppendParams& p, CacheKind kind, bool bf16, int head_dim,
                         hipStream_t s) {
  if (p.num_tokens == 0) return hipSuccess;
  if (head_dim == 128) return bf16 ? dispatch_kind<128, true>(p, kind, s) : dispatch_kind<128, false>(p, kind, s);
  return bf16 ? dispatch_kind<64, true>(p, kind, s) : dispatch_kind<64, false>(p, kind, s);
}

}  // namespace pkv

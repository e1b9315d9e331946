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
#include "launch.h"
#include "common.cuh"
#include "fp8_quant.cuh"

namespace pkv {

template <bool BF16>
__device__ __forceinline__ void widen8(const uint4& x, float (&f)[8]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = h_lo<BF16>(w[i]);
    f[2 * i + 1] = h_hi<BF16>(w[i]);
  }
}

// fp8 row: s = absmax / 448 (1 for an all-zero row), code = RNE_e4m3fn(clamp(x / s, +-448)).
// With a caller-given scale (given, launch-uniform) s is read instead, never written, and the
// quotient is the full division.
template <int LPR, bool BF16>
__device__ __forceinline__ void store_fp8_row(const uint4& x, uint8_t* dst, float* meta, int c,
                                              bool given) {
  float f[8];
  widen8<BF16>(x, f);
  float y[8];
  Fp8RowScale q;
  if (given) {
    q.s = *meta;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fp8_scaled_div(f[e], q);
  } else {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(f[e]));
    q = fp8_row_scale(group_max<LPR>(a));
    // fp8_scaled per value, with the rare full-division rows handled in one wave-uniform branch
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fp8_scaled_fast(f[e], q);
    if (__builtin_amdgcn_ballot_w64(!q.fast) != 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!q.fast) y[e] = fp8_scaled_div(f[e], q);
    }
  }
  // the codes are written with the non-temporal hint (measured on the mixed fp8 append: +6 %)
  typedef uint32_t u32x2_st __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store((u32x2_st){fp8_pack4(y[0], y[1], y[2], y[3]), fp8_pack4(y[4], y[5], y[6], y[7])},
                              reinterpret_cast<u32x2_st*>(dst));
  if (c == 0 && !given) *meta = q.s;
}

// e5m2 / int8 row: s = absmax / M (M = 57344 or 127; 1 for an all-zero row) or the caller's
// scale (given), y = clamp(x / s, +-M) with the correctly rounded quotient, then the format's
// cast (fp8_quant.cuh).
template <int LPR, bool BF16, CacheKind KIND>
__device__ __forceinline__ void store_code_row(const uint4& x, uint8_t* dst, float* meta, int c,
                                               bool given) {
  constexpr float M = KIND == CacheKind::E5m2 ? 57344.f : 127.f;
  float f[8];
  widen8<BF16>(x, f);
  float s;
  if (given) {
    s = *meta;
  } else {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(f[e]));
    a = group_max<LPR>(a);
    s = (a == 0.f) ? 1.f : a / M;
  }
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(f[e] / s, -M), M);
  typedef uint32_t u32x2_st __attribute__((ext_vector_type(2)));
  u32x2_st w;
  if constexpr (KIND == CacheKind::E5m2) {
    w = (u32x2_st){e5m2_pack4(y[0], y[1], y[2], y[3]), e5m2_pack4(y[4], y[5], y[6], y[7])};
  } else {
    w = (u32x2_st){i8_pack4(y[0], y[1], y[2], y[3]), i8_pack4(y[4], y[5], y[6], y[7])};
  }
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2_st*>(dst));
  if (c == 0 && !given) *meta = s;
}

// u3 row: min/max affine parameters in fp32 rounded to fp16, codes clamp(rint(x/s + z), 0, 7),
// 8 codes per lane = one 24-bit octet; each quad of lanes (32 values) writes 3 words.
template <int LPR, bool BF16>
__device__ __forceinline__ void store_u3_row(const uint4& x, uint32_t* dst_row, uint32_t* meta,
                                             int c) {
#pragma clang fp contract(off)
  float f[8];
  widen8<BF16>(x, f);
  float lo = f[0], hi = f[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    lo = fminf(lo, f[e]);
    hi = fmaxf(hi, f[e]);
  }
  lo = group_min<LPR>(lo);
  hi = group_max<LPR>(hi);
  _Float16 s16 = (_Float16)((hi - lo) / 7.0f);
  float s = (float)s16;
  _Float16 z16 = (_Float16)(-lo / s);
  const bool bad = (s == 0.f) || !__builtin_isfinite(s) || !__builtin_isfinite((float)z16);
  if (bad) {
    s16 = (_Float16)1.0f;
    s = 1.0f;
    z16 = (_Float16)(-lo);
  }
  const float z = (float)z16;
  uint32_t o = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = f[e] / s + z;
    const float qf = fminf(fmaxf(__builtin_rintf(t), 0.f), 7.f);
    o |= (uint32_t)qf << (3 * e);
  }
  // word j of the lane's group of 32 values: bytes 4j..4j+3 of four consecutive octets
  const uint32_t next = dpp_u<DPP_QUAD_NEXT>(o);
  const int j = c & 3;
  if (j < 3) dst_row[(c >> 2) * 3 + j] = (o >> (8 * j)) | (next << (24 - 8 * j));
  if (c == 0)
    *meta = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
            ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
}

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
    if constexpr (KIND == CacheKind::Same) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.k_cache) + crow + c * 8) = kx[k];
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.v_cache) + crow + c * 8) = vx[k];
    } else if constexpr (KIND == CacheKind::Fp8) {
      store_fp8_row<LPR, BF16>(kx[k], static_cast<uint8_t*>(p.k_cache) + crow + c * 8,
                               static_cast<float*>(p.k_meta) + mrow, c, p.given_scale != 0);
      store_fp8_row<LPR, BF16>(vx[k], static_cast<uint8_t*>(p.v_cache) + crow + c * 8,
                               static_cast<float*>(p.v_meta) + mrow, c, p.given_scale != 0);
    } else if constexpr (byte_kind(KIND)) {
      store_code_row<LPR, BF16, KIND>(kx[k], static_cast<uint8_t*>(p.k_cache) + crow + c * 8,
                                      static_cast<float*>(p.k_meta) + mrow, c, p.given_scale != 0);
      store_code_row<LPR, BF16, KIND>(vx[k], static_cast<uint8_t*>(p.v_cache) + crow + c * 8,
                                      static_cast<float*>(p.v_meta) + mrow, c, p.given_scale != 0);
    } else {
      store_u3_row<LPR, BF16>(kx[k], static_cast<uint32_t*>(p.k_cache) + crow,
                              static_cast<uint32_t*>(p.k_meta) + mrow, c);
      store_u3_row<LPR, BF16>(vx[k], static_cast<uint32_t*>(p.v_cache) + crow,
                              static_cast<uint32_t*>(p.v_meta) + mrow, c);
    }
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

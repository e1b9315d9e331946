// One (token, kv head) row of the append: the D/8 lanes of the row each hold 8 consecutive
// elements of the new K and V rows and write them into the pool in the cache's format.  Shared by
// kv_append (append.hip) and by the decode kernel's fused append of a decode step's new tokens.
//
// "Write Triton Kv Cache Append Kernel", Required reasoning process steps 4-8: quantised caches
// divide by the scale in fp32 and only then convert (fp8 e4m3fn, fp8 e5m2 and int8 arithmetic in
// fp8_quant.cuh).  The 3-bit cache follows "triton-3bit-kv-cache-kernel" README, sections 1A/1B
// (bit layout) and section 2 test 3 (fp16 affine scale and zero).
#pragma once
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

// Converts and stores the K and V rows of one (token, kv head) row: crow / mrow are the cache
// row and meta entry of its slot (elements of the cache, entries of the meta pools); with given
// scales (byte codes) the meta entries are the caller's scales, read and never written.
template <int LPR, bool BF16, CacheKind KIND>
__device__ __forceinline__ void store_kv_row(const uint4& kx, const uint4& vx, void* k_cache, void* v_cache,
                                             void* k_meta, void* v_meta, int64_t crow, int64_t mrow, int c,
                                             bool given) {
  if constexpr (KIND == CacheKind::Same) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(k_cache) + crow + c * 8) = kx;
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(v_cache) + crow + c * 8) = vx;
  } else if constexpr (KIND == CacheKind::Fp8) {
    store_fp8_row<LPR, BF16>(kx, static_cast<uint8_t*>(k_cache) + crow + c * 8, static_cast<float*>(k_meta) + mrow,
                             c, given);
    store_fp8_row<LPR, BF16>(vx, static_cast<uint8_t*>(v_cache) + crow + c * 8, static_cast<float*>(v_meta) + mrow,
                             c, given);
  } else if constexpr (byte_kind(KIND)) {
    store_code_row<LPR, BF16, KIND>(kx, static_cast<uint8_t*>(k_cache) + crow + c * 8,
                                    static_cast<float*>(k_meta) + mrow, c, given);
    store_code_row<LPR, BF16, KIND>(vx, static_cast<uint8_t*>(v_cache) + crow + c * 8,
                                    static_cast<float*>(v_meta) + mrow, c, given);
  } else {
    store_u3_row<LPR, BF16>(kx, static_cast<uint32_t*>(k_cache) + crow, static_cast<uint32_t*>(k_meta) + mrow, c);
    store_u3_row<LPR, BF16>(vx, static_cast<uint32_t*>(v_cache) + crow, static_cast<uint32_t*>(v_meta) + mrow, c);
  }
}

}  // namespace pkv

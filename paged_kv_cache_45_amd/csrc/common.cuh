// Device helpers shared by the paged KV-cache kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// ---------------------------------------------------------------------------------
// 16-bit float <-> fp32.  Widening is exact; narrowing rounds to nearest even.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <bool BF16>
__device__ __forceinline__ float h_lo(uint32_t w) { return BF16 ? bf16_lo(w) : f16_lo(w); }
template <bool BF16>
__device__ __forceinline__ float h_hi(uint32_t w) { return BF16 ? bf16_hi(w) : f16_hi(w); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                 // round to nearest even
  return u >> 16;
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);      // v_cvt_f16_f32, RNE
}
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return BF16 ? (f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16))
              : (f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16));
}

// Two-element dot product of packed 16-bit pairs accumulated in fp32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Loads of data that is read once (the decode's K/V stream, the append's new rows): the
// non-temporal hint (`nt`) lets the caches stream it instead of allocating it as reusable.
// Measured on the Llama-8B decode step, whose pools far exceed the caches: 118 -> 103 us.
// (Not used where the data was just written and is read back from the caches, as in the
// pack3 -> unpack3 round trip: there it was slower.)
__device__ __forceinline__ uint4 load_stream_u4(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream_u2(const void* p) {
  typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
  const u32x2_nt v = __builtin_nontemporal_load(static_cast<const u32x2_nt*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load_stream_u32(const void* p) {
  return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}
// Buffer loads: a raw buffer resource (stride 0) over the 2^31 - 1 bytes from a wave-uniform
// base, kept in scalar registers, plus a 32-bit per-lane byte offset and a wave-uniform byte
// offset (soffset): no per-lane 64-bit address arithmetic.  Word 3 of the descriptor is the
// gfx9 value for untyped dword access.  `nt` marks data read once (as load_stream_*).
// A resource of 0 records makes every load through it return zeros without a memory access:
// loads that must be issued on every path (so that the wait counts stay exact) but whose data
// is not needed use one.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc buf_rsrc(const void* base, int num_records = 0x7fffffff) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_records, 0x00020000);
}
template <bool NT>
__device__ __forceinline__ uint4 buf_load_u4(BufRsrc r, uint32_t voff, uint32_t soff) {
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, NT ? 2 : 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
template <bool NT>
__device__ __forceinline__ uint2 buf_load_u2(BufRsrc r, uint32_t voff, uint32_t soff) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  const i32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, NT ? 2 : 0);
  return make_uint2((uint32_t)v.x, (uint32_t)v.y);
}
template <bool NT>
__device__ __forceinline__ uint32_t buf_load_u32(BufRsrc r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, NT ? 2 : 0);
}

// Matrix-core product of 16 independent 4x4x4 blocks (v_mfma_f32_4x4x4{f16,bf16_1k}): block b
// (lanes 4b .. 4b + 3) takes A[m][k] from element k of lane 4b + m, B[k][n] from element k of
// lane 4b + n, and adds C[m][n] to register m of lane 4b + n.  The four 16-bit elements of a
// lane's operand are the pairs (a0, a1), resp. (b0, b1), low half first.
template <bool BF16>
__device__ __forceinline__ f32x4_t mfma4x4x4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                              f32x4_t c) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t a = {a0, a1}, b = {b0, b1};
  if constexpr (BF16) {
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                  __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  } else {
    typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4_t, a),
                                              __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
}

template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
  }
}

// ---------------------------------------------------------------------------------
// Cross-lane reductions inside a DPP row (16 lanes).  Every lane of the group gets
// the result.  Group sizes 4, 8 and 16 must be aligned to the group size.
// ---------------------------------------------------------------------------------
enum : int {
  DPP_QUAD_XOR1 = 0xB1,      // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,      // quad_perm [2,3,0,1]
  DPP_QUAD_NEXT = 0xF9,      // quad_perm [1,2,3,3]: lane j reads lane j+1 of its quad
  DPP_ROW_HALF_MIRROR = 0x141,
  DPP_ROW_MIRROR = 0x140,
  DPP_ROW_ROR4 = 0x124,      // lane i of a 16-lane row reads lane (i + 4) mod 16
  DPP_ROW_ROR8 = 0x128,      // lane i of a 16-lane row reads lane (i + 8) mod 16
};
// quad_perm [g, g, g, g]: every lane of a quad reads lane g of the quad
template <int g> constexpr int dpp_quad_bcast() { return g | (g << 2) | (g << 4) | (g << 6); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  x += dpp_f<DPP_QUAD_XOR1>(x);
  x += dpp_f<DPP_QUAD_XOR2>(x);
  if constexpr (N >= 8) x += dpp_f<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp_f<DPP_ROW_MIRROR>(x);
  return x;
}
// group_sum of K independent values, one butterfly stage at a time over all of them: the DPP
// reads of a stage then never wait on the result of the instruction just before them.
template <int N, int K>
__device__ __forceinline__ void group_sum_n(float (&x)[K]) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
#pragma unroll
  for (int k = 0; k < K; ++k) x[k] += dpp_f<DPP_QUAD_XOR1>(x[k]);
#pragma unroll
  for (int k = 0; k < K; ++k) x[k] += dpp_f<DPP_QUAD_XOR2>(x[k]);
  if constexpr (N >= 8) {
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] += dpp_f<DPP_ROW_HALF_MIRROR>(x[k]);
  }
  if constexpr (N >= 16) {
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] += dpp_f<DPP_ROW_MIRROR>(x[k]);
  }
}
template <int N>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dpp_f<DPP_QUAD_XOR1>(x));
  x = fmaxf(x, dpp_f<DPP_QUAD_XOR2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_f<DPP_ROW_HALF_MIRROR>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_f<DPP_ROW_MIRROR>(x));
  return x;
}
template <int N>
__device__ __forceinline__ float group_min(float x) {
  x = fminf(x, dpp_f<DPP_QUAD_XOR1>(x));
  x = fminf(x, dpp_f<DPP_QUAD_XOR2>(x));
  if constexpr (N >= 8) x = fminf(x, dpp_f<DPP_ROW_HALF_MIRROR>(x));
  if constexpr (N >= 16) x = fminf(x, dpp_f<DPP_ROW_MIRROR>(x));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x of lane i ^ 4 (ds_swizzle in bit-mask mode: and 0x1f, or 0, xor 4; no address register)
__device__ __forceinline__ float swz_xor4(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
}

// Sum of the quads of a row of N lanes (16: four quads, 8: two), each lane keeping its place in
// its quad.  For 16 lanes, rotating by 8 and then by 4 adds the same pairs in every quad,
// (x0 + x2) + (x1 + x3) up to the order of each addition's operands, so every quad of the row
// gets the bit-identical sum.
template <int N>
__device__ __forceinline__ float row_quads_sum(float x) {
  static_assert(N == 8 || N == 16, "rows of 8 or 16 lanes");
  if constexpr (N == 16) {
    x += dpp_f<DPP_ROW_ROR8>(x);
    x += dpp_f<DPP_ROW_ROR4>(x);
  } else {
    x += swz_xor4(x);
  }
  return x;
}

}  // namespace pkv

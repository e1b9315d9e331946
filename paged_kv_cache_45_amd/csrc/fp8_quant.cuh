// Byte-code caches: the fp8 e4m3fn quantisation arithmetic of one cache row, the e5m2 and
// int8 casts, and the decode's code-to-value conversions for all three.
//
// "Write Triton Kv Cache Append Kernel", Required reasoning process step 6 and Failure modes:
// each value is divided by the row's scale in fp32 before it is cast, and the cast saturates
// (here: clamp to +-448 first).  The format is OCP E4M3 finite-only (bias 7, max 448), rounded
// to nearest even.
//
// Two shortcuts keep this cheap on gfx950, both checked exhaustively against the plain
// definitions (tests/gpu_kernels/fp8_checks.hip, run by tests/test_gpu_fp8_exhaustive.py):
//  * the quotient x / s of a whole row comes from one correctly rounded reciprocal r = 1 / s
//    and one fma correction per value, q = fma(fma(-s, x r, x), r, x r) with the sign of x:
//    the residual-correction step of Markstein's fma division (P. Markstein, IBM J. Res. Dev.
//    34(1), 1990; J.-M. Muller et al., Handbook of Floating-Point Arithmetic, on division with
//    an fma), here without the theorem's conditions on r and x r, hence the exhaustive check.
//    q can differ from the correctly rounded x / s in its last bit, but for every 16-bit (fp16
//    or bf16) x with |x| <= absmax and every 16-bit absmax, its e4m3 code is the code of the
//    correctly rounded quotient.  Scales outside [2^-100, 2^100] (reciprocal overflow,
//    subnormal products) take the full division.
//  * the cast is v_cvt_pk_fp8_f32 (two values per instruction, OCP E4M3 on gfx950, RNE under
//    the default rounding mode), which equals the integer round-to-nearest-even encoder for
//    every fp32 value in [-448, 448], and torch's CPU float8_e4m3fn cast.
#pragma once
#include <stdint.h>

namespace pkv {

struct Fp8RowScale {
  float s;      // the stored scale: absmax / 448, or 1 for an all-zero row
  float r;      // 1 / s, correctly rounded
  bool fast;    // the one-reciprocal quotient applies
};

__device__ __forceinline__ Fp8RowScale fp8_row_scale(float absmax) {
  Fp8RowScale q;
  q.s = (absmax == 0.f) ? 1.f : absmax / 448.f;
  q.r = 1.f / q.s;
  q.fast = q.s >= 0x1p-100f && q.s <= 0x1p100f;
  return q;
}

// clamp(x / s, -448, 448) through the reciprocal (valid when q.fast) ...
__device__ __forceinline__ float fp8_scaled_fast(float x, const Fp8RowScale& q) {
  const float y0 = x * q.r;
  const float y = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q.s, y0, x), q.r, y0), x);
  return fminf(fmaxf(y, -448.f), 448.f);
}
// ... and through a full division (always valid)
__device__ __forceinline__ float fp8_scaled_div(float x, const Fp8RowScale& q) {
  return fminf(fmaxf(x / q.s, -448.f), 448.f);
}
// the value the append kernel stores the code of
__device__ __forceinline__ float fp8_scaled(float x, const Fp8RowScale& q) {
  return q.fast ? fp8_scaled_fast(x, q) : fp8_scaled_div(x, q);
}

// e4m3fn codes of four clamped values, byte j = code of y_j.
__device__ __forceinline__ uint32_t fp8_pack4(float y0, float y1, float y2, float y3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
  return (uint32_t)w;
}

// ---- read side: e4m3fn codes back to values, exactly.  Every e4m3fn value (|v| <= 448,
// multiples of 2^-9 at the bottom) is exactly a bf16, an fp16 and an fp32 value, so these
// conversions are exact; the row's scale is applied separately by the caller.
typedef __bf16 pkv_bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 pkv_f16x2_t __attribute__((ext_vector_type(2)));

// codes in bytes 2 HI and 2 HI + 1 of w -> a packed pair of 16-bit values (bf16 or fp16)
template <bool BF16, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_16(uint32_t w) {
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
}
// codes in bytes 2 HI and 2 HI + 1 of w -> two fp32 values
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& lo, float& hi) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
  lo = v[0];
  hi = v[1];
}

// ---- e5m2 and int8 caches ("Write Triton Kv Cache Append Kernel", Inputs item 4 and step 6:
// fp8 may also be e5m2, and the cache may be int8).  Both take a per-row scale
// s = absmax / max (max = 57344 for e5m2, 127 for int8; 1 for an all-zero row) and the
// correctly rounded quotient x / s, clamped to +-max.
//  * e5m2 (OCP E5M2: bias 15, 2 mantissa bits, max finite 57344): v_cvt_pk_bf8_f32 is the OCP
//    format on gfx950 and rounds to nearest even; for clamped inputs it equals the integer RNE
//    encoder (checked for every fp32 value in [-57344, 57344]).
//  * int8: round half to even (v_rndne_f32), so the codes lie in [-127, 127].
__device__ __forceinline__ uint32_t e5m2_pack4(float y0, float y1, float y2, float y3) {
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(y2, y3, w, true);
  return (uint32_t)w;
}
__device__ __forceinline__ uint32_t i8_pack4(float y0, float y1, float y2, float y3) {
  const uint32_t b0 = (uint32_t)(int)__builtin_rintf(y0) & 0xffu;
  const uint32_t b1 = (uint32_t)(int)__builtin_rintf(y1) & 0xffu;
  const uint32_t b2 = (uint32_t)(int)__builtin_rintf(y2) & 0xffu;
  const uint32_t b3 = (uint32_t)(int)__builtin_rintf(y3) & 0xffu;
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// Read side.  Every e5m2 value is exactly an fp16, a bf16 and an fp32 value (fp16 shares its
// exponent range; an e5m2 code is the upper byte of the fp16 encoding), and every int8 value
// has at most 8 significant bits, so these conversions are exact as well.
template <bool BF16, bool HI>
__device__ __forceinline__ uint32_t e5m2x2_to_16(uint32_t w) {
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, HI));
  }
}
template <bool HI>
__device__ __forceinline__ void e5m2x2_to_f32(uint32_t w, float& lo, float& hi) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_bf8(w, HI);
  lo = v[0];
  hi = v[1];
}
// int8 codes in bytes 2 HI and 2 HI + 1 of w, sign-extended and converted to fp32
template <bool HI>
__device__ __forceinline__ void i8x2_to_f32(uint32_t w, float& lo, float& hi) {
  lo = (float)((int32_t)(w << (HI ? 8 : 24)) >> 24);
  hi = (float)((int32_t)(w << (HI ? 0 : 16)) >> 24);
}
template <bool BF16, bool HI>
__device__ __forceinline__ uint32_t i8x2_to_16(uint32_t w) {
  float lo, hi;
  i8x2_to_f32<HI>(w, lo, hi);
  if constexpr (BF16) {
    // an integer of magnitude <= 128 is exact in bf16: the upper halves of the fp32 values
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  } else {
    // exact in fp16 (|v| <= 2048), so the round-toward-zero pack does not round
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
}

}  // namespace pkv

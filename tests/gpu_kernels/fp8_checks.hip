// Test-only kernels: exhaustive checks of the fp8 quantisation shortcuts, the e5m2 cast and the
// decode's code-to-value conversions (e4m3fn, e5m2, int8) in
// paged_kv_cache_45_amd/csrc/fp8_quant.cuh against their plain definitions.  Built next to
// this file as libpkv_fp8_checks.so by the package build; loaded only by
// tests/test_gpu_fp8_exhaustive.py.  Every kernel writes one count (or one code) per thread
// with a plain store; no atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../paged_kv_cache_45_amd/csrc/fp8_quant.cuh"

namespace {

// Plain integer round-to-nearest-even onto OCP E4M3 (bias 7, max 448) for |y| <= 448: keep 3
// of the 23 mantissa bits of a normal value, rounding the 20 dropped bits half to even (a
// carry may move into the next binade), rebias 127 -> 7; below 2^-6 the values are
// multiples of 2^-9 and y * 2^9 is exact.  The sign of zero is kept.
__device__ uint32_t e4m3fn_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x3C800000u) {
    code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return code | sign;
}

__device__ float widen16(uint32_t h, bool bf16) {
  return bf16 ? __uint_as_float(h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Magnitudes u = t * 256 + j (j < 256) with u <= 448's bit pattern: codes[u] = hardware code
// of +y; bad[t] counts values whose hardware code differs from e4m3fn_rne, for +y or -y.
__global__ void hw_codes(uint32_t u0, uint32_t n_threads, uint8_t* codes, uint32_t* bad) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_threads) return;
  uint32_t nbad = 0;
  for (uint32_t j = 0; j < 256; ++j) {
    const uint32_t u = u0 + t * 256u + j;
    if (u > 0x43E00000u) break;
    const float y = __uint_as_float(u);
    const uint32_t cp = pkv::fp8_pack4(y, -y, 0.f, 0.f);
    if ((cp & 0xffu) != e4m3fn_rne(y) || ((cp >> 8) & 0xffu) != e4m3fn_rne(-y)) ++nbad;
    codes[t * 256u + j] = (uint8_t)(cp & 0xffu);
  }
  bad[t] = nbad;
}

// One block per 16-bit absmax pattern a (positive); every 16-bit x with |x| <= a: the code of
// fp8_scaled(x) (the kernel's quotient) vs the code of clamp(x / s) with a full division.
__global__ void quotient_codes(int bf16, uint32_t* bad) {
  const float a = widen16(blockIdx.x, bf16 != 0);
  uint32_t nbad = 0;
  if (a > 0.f && __builtin_isfinite(a)) {
    const pkv::Fp8RowScale q = pkv::fp8_row_scale(a);
    for (uint32_t xh = threadIdx.x; xh < 65536u; xh += blockDim.x) {
      const float x = widen16(xh, bf16 != 0);
      if (!(__builtin_fabsf(x) <= a)) continue;
      const float want = fminf(fmaxf(x / q.s, -448.f), 448.f);
      if (e4m3fn_rne(pkv::fp8_scaled(x, q)) != e4m3fn_rne(want)) ++nbad;
    }
  }
  bad[blockIdx.x * blockDim.x + threadIdx.x] = nbad;
}

// The decode's code-to-value conversions, for every code c: thread c converts the word
// c * 0x01010101 with both byte-pair selects.  out16[4c + 0..1] = bf16 pairs (low, high
// select), out16[4c + 2..3] = fp16 pairs; out32[4c + 0..3] = fp32 values (low pair, high pair).
__global__ void dequant_codes(uint32_t* out16, float* out32) {
  const uint32_t c = threadIdx.x;
  const uint32_t w = c * 0x01010101u;
  out16[4 * c + 0] = pkv::fp8x2_to_16<true, false>(w);
  out16[4 * c + 1] = pkv::fp8x2_to_16<true, true>(w);
  out16[4 * c + 2] = pkv::fp8x2_to_16<false, false>(w);
  out16[4 * c + 3] = pkv::fp8x2_to_16<false, true>(w);
  float a, b;
  pkv::fp8x2_to_f32<false>(w, a, b);
  out32[4 * c + 0] = a;
  out32[4 * c + 1] = b;
  pkv::fp8x2_to_f32<true>(w, a, b);
  out32[4 * c + 2] = a;
  out32[4 * c + 3] = b;
}

// Plain integer round-to-nearest-even onto OCP E5M2 (bias 15, max 57344) for |y| <= 57344:
// keep 2 of the 23 mantissa bits of a normal value, rounding the 21 dropped bits half to even,
// rebias 127 -> 15; below 2^-14 the values are multiples of 2^-16 and y * 2^16 is exact.
__device__ uint32_t e5m2_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x38800000u) {
    code = ((a + 0xFFFFFu + ((a >> 21) & 1u)) >> 21) - (112u << 2);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 65536.0f);
  }
  return code | sign;
}

// As hw_codes, for the e5m2 cast and magnitudes up to 57344's bit pattern.
__global__ void hw_codes_e5m2(uint32_t u0, uint32_t n_threads, uint8_t* codes, uint32_t* bad) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_threads) return;
  uint32_t nbad = 0;
  for (uint32_t j = 0; j < 256; ++j) {
    const uint32_t u = u0 + t * 256u + j;
    if (u > 0x47600000u) break;
    const float y = __uint_as_float(u);
    const uint32_t cp = pkv::e5m2_pack4(y, -y, 0.f, 0.f);
    if ((cp & 0xffu) != e5m2_rne(y) || ((cp >> 8) & 0xffu) != e5m2_rne(-y)) ++nbad;
    codes[t * 256u + j] = (uint8_t)(cp & 0xffu);
  }
  bad[t] = nbad;
}

// The e5m2 and int8 read-side conversions, laid out as dequant_codes: fmt 0 = e5m2, 1 = int8.
__global__ void dequant_codes_byte(int fmt, uint32_t* out16, float* out32) {
  const uint32_t c = threadIdx.x;
  const uint32_t w = c * 0x01010101u;
  float a, b, x, y;
  if (fmt == 0) {
    out16[4 * c + 0] = pkv::e5m2x2_to_16<true, false>(w);
    out16[4 * c + 1] = pkv::e5m2x2_to_16<true, true>(w);
    out16[4 * c + 2] = pkv::e5m2x2_to_16<false, false>(w);
    out16[4 * c + 3] = pkv::e5m2x2_to_16<false, true>(w);
    pkv::e5m2x2_to_f32<false>(w, a, b);
    pkv::e5m2x2_to_f32<true>(w, x, y);
  } else {
    out16[4 * c + 0] = pkv::i8x2_to_16<true, false>(w);
    out16[4 * c + 1] = pkv::i8x2_to_16<true, true>(w);
    out16[4 * c + 2] = pkv::i8x2_to_16<false, false>(w);
    out16[4 * c + 3] = pkv::i8x2_to_16<false, true>(w);
    pkv::i8x2_to_f32<false>(w, a, b);
    pkv::i8x2_to_f32<true>(w, x, y);
  }
  out32[4 * c + 0] = a;
  out32[4 * c + 1] = b;
  out32[4 * c + 2] = x;
  out32[4 * c + 3] = y;
}

}  // namespace

extern "C" int fp8chk_hw_codes_e5m2(uint32_t u0, uint32_t n_threads, uint8_t* codes, uint32_t* bad,
                                    hipStream_t s) {
  hipLaunchKernelGGL(hw_codes_e5m2, dim3((n_threads + 255) / 256), dim3(256), 0, s, u0, n_threads, codes,
                     bad);
  return (int)hipGetLastError();
}

extern "C" int fp8chk_dequant_codes_byte(int fmt, uint32_t* out16, float* out32, hipStream_t s) {
  hipLaunchKernelGGL(dequant_codes_byte, dim3(1), dim3(256), 0, s, fmt, out16, out32);
  return (int)hipGetLastError();
}

extern "C" int fp8chk_dequant_codes(uint32_t* out16, float* out32, hipStream_t s) {
  hipLaunchKernelGGL(dequant_codes, dim3(1), dim3(256), 0, s, out16, out32);
  return (int)hipGetLastError();
}

extern "C" int fp8chk_hw_codes(uint32_t u0, uint32_t n_threads, uint8_t* codes, uint32_t* bad,
                               hipStream_t s) {
  hipLaunchKernelGGL(hw_codes, dim3((n_threads + 255) / 256), dim3(256), 0, s, u0, n_threads, codes, bad);
  return (int)hipGetLastError();
}

extern "C" int fp8chk_quotient_codes(int bf16, uint32_t* bad, hipStream_t s) {
  hipLaunchKernelGGL(quotient_codes, dim3(32768), dim3(256), 0, s, bf16, bad);
  return (int)hipGetLastError();
}

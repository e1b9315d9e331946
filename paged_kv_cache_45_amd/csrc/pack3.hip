// 3-bit packing kernels.
//
// Layout ("triton-3bit-kv-cache-kernel" README, sections 1A and 1B): value j of each
// group of 8 occupies bits 3j..3j+2 of a little-endian 24-bit octet; 32 values fill
// three little-endian uint32 words, lane i at bit 3i, lanes 10 and 21 crossing a
// word boundary.
//
// Fast path: one thread per group of 32 values (32 bytes in as two 16-byte loads,
// 12 bytes out as three dwords), used when `values` is 16-byte aligned and `packed`
// 4-byte aligned.  Trailing groups of 8 values, and unaligned buffers, take the
// octet path (one thread per octet, byte accesses).
#include "launch.h"
#include "common.cuh"

namespace pkv {

// 8 bytes of values (two dwords, value j in byte j) -> 24-bit octet.
__device__ __forceinline__ uint32_t octet_from_bytes(uint32_t lo, uint32_t hi) {
  uint32_t o = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o |= ((lo >> (8 * j)) & 7u) << (3 * j);
    o |= ((hi >> (8 * j)) & 7u) << (3 * (j + 4));
  }
  return o;
}

// 24-bit octet -> 8 bytes of values (two dwords).
__device__ __forceinline__ void bytes_from_octet(uint32_t o, uint32_t& lo, uint32_t& hi) {
  lo = 0;
  hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo |= ((o >> (3 * j)) & 7u) << (8 * j);
    hi |= ((o >> (3 * (j + 4))) & 7u) << (8 * j);
  }
}

__global__ __launch_bounds__(256) void pack3_kernel(const uint8_t* __restrict__ values,
                                                    uint8_t* __restrict__ packed, int64_t n_groups32,
                                                    int64_t first_octet, int64_t n_octets) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_groups32) {
    const uint4 a = reinterpret_cast<const uint4*>(values)[2 * i];
    const uint4 b = reinterpret_cast<const uint4*>(values)[2 * i + 1];
    const uint32_t o0 = octet_from_bytes(a.x, a.y), o1 = octet_from_bytes(a.z, a.w);
    const uint32_t o2 = octet_from_bytes(b.x, b.y), o3 = octet_from_bytes(b.z, b.w);
    uint32_t* dst = reinterpret_cast<uint32_t*>(packed) + 3 * i;
    dst[0] = o0 | (o1 << 24);
    dst[1] = (o1 >> 8) | (o2 << 16);
    dst[2] = (o2 >> 16) | (o3 << 8);
    return;
  }
  const int64_t k = first_octet + (i - n_groups32);      // octet path
  if (i >= n_groups32 && k < n_octets) {
    const uint8_t* src = values + 8 * k;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= (uint32_t)src[j] << (8 * j);
      hi |= (uint32_t)src[4 + j] << (8 * j);
    }
    const uint32_t o = octet_from_bytes(lo, hi);
    uint8_t* dst = packed + 3 * k;
    dst[0] = (uint8_t)o;
    dst[1] = (uint8_t)(o >> 8);
    dst[2] = (uint8_t)(o >> 16);
  }
}

__global__ __launch_bounds__(256) void unpack3_kernel(const uint8_t* __restrict__ packed,
                                                      uint8_t* __restrict__ values, int64_t n_groups32,
                                                      int64_t first_octet, int64_t n_octets) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_groups32) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(packed) + 3 * i;
    const uint32_t w0 = src[0], w1 = src[1], w2 = src[2];
    uint4 a, b;
    bytes_from_octet(w0 & 0xffffffu, a.x, a.y);
    bytes_from_octet(((w0 >> 24) | (w1 << 8)) & 0xffffffu, a.z, a.w);
    bytes_from_octet(((w1 >> 16) | (w2 << 16)) & 0xffffffu, b.x, b.y);
    bytes_from_octet(w2 >> 8, b.z, b.w);
    reinterpret_cast<uint4*>(values)[2 * i] = a;
    reinterpret_cast<uint4*>(values)[2 * i + 1] = b;
    return;
  }
  const int64_t k = first_octet + (i - n_groups32);
  if (i >= n_groups32 && k < n_octets) {
    const uint8_t* src = packed + 3 * k;
    const uint32_t o = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16);
    uint32_t lo, hi;
    bytes_from_octet(o, lo, hi);
    uint8_t* dst = values + 8 * k;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[j] = (uint8_t)(lo >> (8 * j));
      dst[4 + j] = (uint8_t)(hi >> (8 * j));
    }
  }
}

static void split_work(const void* vals, const void* pk, int64_t n_values, int64_t& groups,
                       int64_t& first_octet, int64_t& n_octets) {
  n_octets = n_values / 8;
  const bool aligned = ((uintptr_t)vals % 16 == 0) && ((uintptr_t)pk % 4 == 0);
  groups = aligned ? n_values / 32 : 0;
  first_octet = groups * 4;
}

hipError_t launch_pack3(const uint8_t* values, uint8_t* packed, int64_t n_values,
                        hipStream_t stream) {
  int64_t groups, first, n_oct;
  split_work(values, packed, n_values, groups, first, n_oct);
  const int64_t threads = groups + (n_oct - first);
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(pack3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, values, packed,
                     groups, first, n_oct);
  return hipGetLastError();
}

hipError_t launch_unpack3(const uint8_t* packed, uint8_t* values, int64_t n_values,
                          hipStream_t stream) {
  int64_t groups, first, n_oct;
  split_work(values, packed, n_values, groups, first, n_oct);
  const int64_t threads = groups + (n_oct - first);
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(unpack3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, packed, values,
                     groups, first, n_oct);
  return hipGetLastError();
}

}  // namespace pkv

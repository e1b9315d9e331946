// Paged decode attention: the split-K merge kernels and the host side (grid plan, dispatch).
// The decode kernel itself is in decode_kernel.cuh.
#include <algorithm>

#include "decode_kernel.cuh"

namespace pkv {

// One workgroup per (request, kv head, query head of the group): merges the partial states
// of a split segment by log-sum-exp, writes zeros for an empty context, and leaves
// single-workgroup segments alone.  The D / 4 x splits threads (4 consecutive elements each:
// 16-byte partial loads, 8-byte output stores) split the partials `splits` ways (each with
// kMergeBatch loads in flight), then combine through LDS.  4 elements per thread in place of 1:
// long-context merge 7.21 -> 6.72 us, 3-bit decode merge 5.36 -> 5.00 us.
constexpr int kMergeMaxSplit = 8;
constexpr int kMergeBatch = 4;
// elements per thread of merge_vec_kernel (Llama-8B step: merge 5.15 -> 4.51 us with 4, 4.92 with 8)
constexpr int kMergeVec = 4;

template <int D, int G, bool BF16>
__global__ __launch_bounds__(D / 4 * kMergeMaxSplit) void merge_kernel(DecodeParams p) {
  constexpr int TPD = D / 4;                           // threads per split, 4 elements each
  __shared__ float s_m[kMergeMaxSplit][TPD], s_l[kMergeMaxSplit][TPD];
  __shared__ float4 s_a[kMergeMaxSplit][TPD];
  const int kMergeSplit = blockDim.x / TPD;
  const int g = blockIdx.x % G;
  const int kvh = (blockIdx.x / G) % p.num_kv_heads;
  const int b = blockIdx.x / (G * p.num_kv_heads);
  const int hg = kvh / p.heads_per_group, hh = kvh % p.heads_per_group;
  const int t = threadIdx.x % TPD, d = t * 4, part = threadIdx.x / TPD;
  uint16_t* out = static_cast<uint16_t*>(p.out) + b * p.o_sb + (int64_t)(kvh * G + g) * p.o_sh + d;
  // The decode kernel recorded, for this (request, head group) segment, the partial slot of the
  // workgroup w0 that holds its first unit (2 * w0 + 0 if the segment starts w0's range, else
  // 2 * w0 + 1) and the workgroup w1 that holds its last unit; w0 + 1 .. w1 keep theirs in
  // slot 0 (a workgroup with an empty range wrote an empty state there).  The record is loaded
  // together with the context length, not after it (one load latency less: Llama-8B step +0.5 %).
  const int64_t sidx = (int64_t)b * p.num_head_groups + hg;
  const int2 seg = *reinterpret_cast<const int2*>(p.ws_seg + 2 * sidx);
  if (clamp_ctx(p, b) == 0) {
    if (part == 0) *reinterpret_cast<uint2*>(out) = make_uint2(0u, 0u);
    return;
  }
  const int64_t first = seg.x;
  const int64_t w0 = first >> 1, w1 = seg.y;
  if (w0 == w1) return;                                // one workgroup covered it and wrote out
  const int64_t hpg = p.heads_per_group;
  auto slot_of = [&](int64_t j) {        // j-th partial, j = 0 .. w1 - w0
    return ((j == 0 ? first : (w0 + j) * 2) * hpg + hh) * G + g;
  };
  float M = neg_inf(), L = 0.f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t j0 = part; j0 <= w1 - w0; j0 += kMergeSplit * kMergeBatch) {
    float2 ml[kMergeBatch];
    float4 a[kMergeBatch];
    bool ok[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {            // independent loads, all in flight
      const int64_t j = j0 + (int64_t)u * kMergeSplit;
      ok[u] = j <= w1 - w0;
      const int64_t sl = ok[u] ? slot_of(j) : 0;
      ml[u] = ok[u] ? *reinterpret_cast<const float2*>(p.ws_ml + sl * 2) : make_float2(neg_inf(), 0.f);
      a[u] = ok[u] ? *reinterpret_cast<const float4*>(p.ws_acc + sl * D + d) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (!ok[u] || ml[u].x == neg_inf()) continue;    // an empty range's state adds nothing
      const float mn = fmaxf(M, ml[u].x);
      const float fo = fast_exp2(M - mn), fn = fast_exp2(ml[u].x - mn);
      L = L * fo + ml[u].y * fn;
      A.x = A.x * fo + a[u].x * fn;
      A.y = A.y * fo + a[u].y * fn;
      A.z = A.z * fo + a[u].z * fn;
      A.w = A.w * fo + a[u].w * fn;
      M = mn;
    }
  }
  s_m[part][t] = M;
  s_l[part][t] = L;
  s_a[part][t] = A;
  __syncthreads();
  if (part == 0) {
    float Mt = s_m[0][t];
    for (int q = 1; q < kMergeSplit; ++q) Mt = fmaxf(Mt, s_m[q][t]);
    float Lt = 0.f;
    float4 At = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q = 0; q < kMergeSplit; ++q) {
      const float f = fast_exp2(s_m[q][t] - Mt);       // an empty split has m = -inf, f = 0
      Lt += s_l[q][t] * f;
      At.x += s_a[q][t].x * f;
      At.y += s_a[q][t].y * f;
      At.z += s_a[q][t].z * f;
      At.w += s_a[q][t].w * f;
    }
    const float o[4] = {At.x / Lt, At.y / Lt, At.z / Lt, At.w / Lt};
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = BF16 ? f32_to_bf16_bits(o[e]) : f32_to_f16_bits(o[e]);
    *reinterpret_cast<uint2*>(out) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }
}

// The merge where each thread merges all partials of its elements in one pass (few partials per
// segment): one workgroup per (request, kv head) covering the G query heads, kMergeVec
// consecutive elements per thread (16-byte partial loads, 8-byte output stores per 4 elements),
// so that fewer waves are launched than with one element per thread.
template <int D, int G, bool BF16>
__global__ __launch_bounds__(G * D / kMergeVec) void merge_vec_kernel(DecodeParams p) {
  constexpr int V = kMergeVec, NQ = V / 4;             // elements, float4 groups per thread
  constexpr int TPH = D / V;                           // threads per query head
  const int kvh = blockIdx.x % p.num_kv_heads;
  const int b = blockIdx.x / p.num_kv_heads;
  const int g = threadIdx.x / TPH, d = (threadIdx.x % TPH) * V;
  const int hg = kvh / p.heads_per_group, hh = kvh % p.heads_per_group;
  uint16_t* out = static_cast<uint16_t*>(p.out) + b * p.o_sb + (int64_t)(kvh * G + g) * p.o_sh + d;
  const int64_t sidx = (int64_t)b * p.num_head_groups + hg;
  const int2 seg = *reinterpret_cast<const int2*>(p.ws_seg + 2 * sidx);   // as in merge_kernel
  if (clamp_ctx(p, b) == 0) {
#pragma unroll
    for (int k = 0; k < NQ; ++k) reinterpret_cast<uint2*>(out)[k] = make_uint2(0u, 0u);
    return;
  }
  const int64_t first = seg.x;
  const int64_t w0 = first >> 1, w1 = seg.y;
  if (w0 == w1) return;
  const int64_t hpg = p.heads_per_group;
  auto slot_of = [&](int64_t j) { return ((j == 0 ? first : (w0 + j) * 2) * hpg + hh) * G + g; };
  float M = neg_inf(), L = 0.f, A[V];
#pragma unroll
  for (int e = 0; e < V; ++e) A[e] = 0.f;
  for (int64_t j0 = 0; j0 <= w1 - w0; j0 += kMergeBatch) {
    float2 ml[kMergeBatch];
    float4 a[kMergeBatch][NQ];
    bool ok[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {            // independent loads, all in flight
      const int64_t j = j0 + u;
      ok[u] = j <= w1 - w0;
      const int64_t sl = ok[u] ? slot_of(j) : 0;
      ml[u] = ok[u] ? *reinterpret_cast<const float2*>(p.ws_ml + sl * 2) : make_float2(neg_inf(), 0.f);
#pragma unroll
      for (int k = 0; k < NQ; ++k)
        a[u][k] = ok[u] ? reinterpret_cast<const float4*>(p.ws_acc + sl * D + d)[k] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (!ok[u] || ml[u].x == neg_inf()) continue;    // an empty range's state adds nothing
      const float mn = fmaxf(M, ml[u].x);
      const float fo = fast_exp2(M - mn), fn = fast_exp2(ml[u].x - mn);
      L = L * fo + ml[u].y * fn;
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        A[4 * k + 0] = A[4 * k + 0] * fo + a[u][k].x * fn;
        A[4 * k + 1] = A[4 * k + 1] * fo + a[u][k].y * fn;
        A[4 * k + 2] = A[4 * k + 2] * fo + a[u][k].z * fn;
        A[4 * k + 3] = A[4 * k + 3] * fo + a[u][k].w * fn;
      }
      M = mn;
    }
  }
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float o = A[4 * k + e] / L;
      h[e] = BF16 ? f32_to_bf16_bits(o) : f32_to_f16_bits(o);
    }
    reinterpret_cast<uint2*>(out)[k] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }
}

namespace {

int heads_per_instr(int head_dim, int num_kv_heads) {
  const int rpi = 64 / (head_dim / 8);
  int hpi = 1;
  while (hpi * 2 <= rpi && num_kv_heads % (hpi * 2) == 0) hpi *= 2;
  return hpi;
}

const void* decode_kernel_ptr(int head_dim, int group, bool bf16, CacheKind kind, int hpi) {
  const bool d128 = head_dim == 128;
  switch (kind) {
    case CacheKind::U3:
      return d128 ? decode_kernel_ptr_u3_d128(group, bf16, hpi) : decode_kernel_ptr_u3_d64(group, bf16, hpi);
    case CacheKind::Fp8:
      return d128 ? decode_kernel_ptr_fp8_d128(group, bf16, hpi) : decode_kernel_ptr_fp8_d64(group, bf16, hpi);
    case CacheKind::E5m2:
      return d128 ? decode_kernel_ptr_e5m2_d128(group, bf16, hpi) : decode_kernel_ptr_e5m2_d64(group, bf16, hpi);
    case CacheKind::I8:
      return d128 ? decode_kernel_ptr_i8_d128(group, bf16, hpi) : decode_kernel_ptr_i8_d64(group, bf16, hpi);
    default:
      return d128 ? decode_kernel_ptr_same_d128(group, bf16, hpi) : decode_kernel_ptr_same_d64(group, bf16, hpi);
  }
}

const void* merge_kernel_ptr(int head_dim, int group, bool bf16) {
#define PKV_MERGE(DD, GG)                                                                   \
  if (head_dim == DD && group == GG)                                                        \
    return bf16 ? reinterpret_cast<const void*>(&merge_kernel<DD, GG, true>)               \
                : reinterpret_cast<const void*>(&merge_kernel<DD, GG, false>);
  PKV_MERGE(128, 1) PKV_MERGE(128, 2) PKV_MERGE(128, 4) PKV_MERGE(128, 8)
  PKV_MERGE(64, 1) PKV_MERGE(64, 2) PKV_MERGE(64, 4) PKV_MERGE(64, 8)
#undef PKV_MERGE
  return nullptr;
}

const void* merge_vec_kernel_ptr(int head_dim, int group, bool bf16) {
#define PKV_MERGE(DD, GG)                                                                   \
  if (head_dim == DD && group == GG)                                                        \
    return bf16 ? reinterpret_cast<const void*>(&merge_vec_kernel<DD, GG, true>)           \
                : reinterpret_cast<const void*>(&merge_vec_kernel<DD, GG, false>);
  PKV_MERGE(128, 1) PKV_MERGE(128, 2) PKV_MERGE(128, 4) PKV_MERGE(128, 8)
  PKV_MERGE(64, 1) PKV_MERGE(64, 2) PKV_MERGE(64, 4) PKV_MERGE(64, 8)
#undef PKV_MERGE
  return nullptr;
}

int resident_wgs_per_cu(const void* fn, int threads, size_t lds) {
  int n = 0;
  if (!fn || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) != hipSuccess || n <= 0)
    n = 8;                         // no device to ask: assume the most a CU can hold
  return n;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

}  // namespace

DecodePlan plan_decode(int batch, int num_q_heads, int num_kv_heads, int head_dim, int max_context_len,
                       int partition_size, int bf16, int kind) {
  DecodePlan P{};
  P.hpi = heads_per_instr(head_dim, num_kv_heads);
  const int waves = num_kv_heads / P.hpi;        // waves to cover all heads of a token
  int hw = 1;                                    // head waves per workgroup (at most 4)
  for (int w = std::min(waves, 4); w >= 1; --w)
    if (waves % w == 0) { hw = w; break; }
  // token streams: up to 4, within kMaxWaves waves (their chunks are shared out at run time)
  P.token_streams = std::max(1, std::min(4, kMaxWaves / hw));
  P.waves_per_wg = hw * P.token_streams;
  P.heads_per_group = P.hpi * hw;
  {
    const int rpi = 64 / (head_dim / 8), tpi = rpi / P.hpi, ni = std::min(4, 16 / tpi);
    P.chunk_tokens = ni * tpi;
  }
  P.num_head_groups = num_kv_heads / P.heads_per_group;
  const int group = num_q_heads / num_kv_heads;
  P.lds_bytes = (size_t)((batch + 1 + 3) & ~3) * sizeof(int) +
                (size_t)(P.token_streams - 1) * P.heads_per_group * group * (head_dim + 2) * sizeof(float);
  int per_cu = 0;
  for (int bf = 0; bf < 2; ++bf)
    for (int kd = 0; kd < kNumCacheKinds; ++kd) {    // every CacheKind value
      if ((bf16 >= 0 && bf != bf16) || (kind >= 0 && kd != kind)) continue;
      const CacheKind ck = static_cast<CacheKind>(kd);
      per_cu = std::max(per_cu, resident_wgs_per_cu(decode_kernel_ptr(head_dim, group, bf != 0, ck, P.hpi),
                                                    P.waves_per_wg * 64, P.lds_bytes));
    }
  const int64_t units = (int64_t)batch * P.num_head_groups *
                        ((max_context_len + partition_size - 1) / partition_size);
  const int cus = device_cus();
  P.num_wgs = std::min<int64_t>((int64_t)cus * per_cu, std::max<int64_t>(units, 1));
  P.split_tier = std::min<int64_t>(P.num_wgs, cus);
  return P;
}

hipError_t launch_decode(const DecodeParams& p, const DecodePlan& plan, CacheKind kind, bool bf16,
                         int head_dim, int group, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  const void* fn = decode_kernel_ptr(head_dim, group, bf16, kind, plan.hpi);
  const void* mf = merge_kernel_ptr(head_dim, group, bf16);
  const void* mvf = merge_vec_kernel_ptr(head_dim, group, bf16);
  if (!fn || !mf || !mvf) return hipErrorInvalidValue;
  void* args[] = {const_cast<DecodeParams*>(&p)};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)plan.num_wgs), dim3(plan.waves_per_wg * 64), args,
                      plan.lds_bytes, s);
  if (e != hipSuccess) return e;
  // split the partials of a segment so that each thread merges about 2 x kMergeBatch of them;
  // where one split suffices, the one-pass form with several elements per thread
  const int64_t per_seg = plan.num_wgs / std::max<int64_t>(1, (int64_t)p.batch * plan.num_head_groups) + 2;
  int splits = 1;
  while (splits < kMergeMaxSplit && per_seg > (int64_t)splits * 2 * kMergeBatch) splits *= 2;
  if (splits == 1)
    e = hipLaunchKernel(mvf, dim3((unsigned)(p.batch * p.num_kv_heads)), dim3(group * head_dim / kMergeVec), args, 0, s);
  else
    e = hipLaunchKernel(mf, dim3((unsigned)(p.batch * p.num_kv_heads * group)), dim3(head_dim / 4 * splits),
                        args, 0, s);
  return e != hipSuccess ? e : hipGetLastError();
}

int auto_partition_size(int, int, int) { return 16; }

}  // namespace pkv

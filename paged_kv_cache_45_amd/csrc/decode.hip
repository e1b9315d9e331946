// Paged decode attention (one query token per request) with split-K partitions.
//
// What is computed ("Triton KV Cache and PagedAttention", Step 1 and the reference
// answer, TODO 1-5): for request b and query head h, out = sum_t softmax_t(sm_scale *
// q.k_t) v_t over the first context_lens[b] tokens; token t lives in physical block
// block_tables[b, t / block_size] at slot t % block_size; tokens past the context are
// masked; the softmax is accumulated online (running max m, running sum l, unnormalised
// accumulator).  GQA ("Write Triton Kv Cache Append Kernel", Kernel design rules): the G =
// Hq / Hkv query heads h = kvh*G .. kvh*G+G-1 share kv head kvh.  The 3-bit cache
// ("triton-3bit-kv-cache-kernel" README, title paragraph and section 2) is unpacked and
// dequantised, x = (q - z) * s, in registers.
//
// MI355X mapping:
//  * one 4-wave workgroup per (kv head, request, partition), kv head fastest in the
//    flattened grid (balances the XCDs); the workgroup owns the token range
//    [partition * P, (partition + 1) * P) of one (request, kv head) and all G query heads
//    of that kv head, so every K/V byte is read from HBM once.
//  * The range is cut into 16-token chunks (a block holds 1, 2 or 4 of them); wave w takes
//    chunks w, w+4, ...  The physical block of each of a wave's chunks is fetched once up
//    front into one VGPR (lane k = k-th chunk) and read back with v_readlane.
//  * Lane layout: D/8 lanes per token row, each lane owning 8 consecutive elements
//    (16 bytes of K and of V, one global_load_dwordx4 each); a wave instruction covers
//    4 (D = 128) or 8 (D = 64) token rows.
//  * QK: v_dot2_f32_{bf16,f16} on the packed pairs, then a DPP reduction inside the lane
//    group; every lane of a row ends with the row's scores for all G heads.
//  * Each token row keeps its own online-softmax state (m, l in log2 units, and the
//    lane's 8 accumulator columns per head); rows are merged with shuffles at the end,
//    the 4 waves through LDS.
//  * Partitions of one request are merged by log-sum-exp in a second small kernel; a
//    request that fits in one partition writes its output directly.
#include "launch.h"
#include "common.cuh"

namespace pkv {

constexpr int kWaves = 4;           // waves per workgroup
constexpr int kChunk = 16;          // tokens per chunk

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// Combine two online-softmax states (m in log2 units).  Returns the factors that scale
// each side's (l, acc) to the common maximum.
__device__ __forceinline__ void lse_factors(float ma, float mb, float& m, float& fa, float& fb) {
  m = fmaxf(ma, mb);
  const float mu = (m == neg_inf()) ? 0.f : m;
  fa = fast_exp2(ma - mu);
  fb = fast_exp2(mb - mu);
}

template <int D, int G, bool BF16, CacheKind KIND>
__global__ __launch_bounds__(kWaves * 64) void decode_kernel(DecodeParams p) {
  constexpr int LPR = D / 8;           // lanes per token row
  constexpr int RPI = 64 / LPR;        // token rows per wave instruction
  constexpr int NI = kChunk / RPI;     // wave instructions per chunk
  static_assert(KIND == CacheKind::Same || KIND == CacheKind::U3, "decode cache kind");

  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = lane / LPR;
  const int c = lane % LPR;
  // Flattened grid, kv head fastest: consecutive workgroup ids go round-robin to the 8 XCDs,
  // so with Hkv = 8 each XCD owns one kv head of every (request, partition) and all XCDs
  // get the same work; partitions vary slowest, so the mostly-empty high partitions of
  // short requests come last.
  const int64_t wg = blockIdx.x;
  const int kvh = (int)(wg % p.num_kv_heads);
  const int b = (int)((wg / p.num_kv_heads) % p.batch);
  const int part = (int)(wg / ((int64_t)p.num_kv_heads * p.batch));
  const int h0 = kvh * G;
  // out-of-contract lengths are clamped so that no access leaves the grid's buffers
  const int ctx = min(max(p.context_lens[b], 0), p.max_context_len);
  const int nparts = (ctx + p.partition_size - 1) / p.partition_size;

  if (part >= nparts) {
    if (part == 0) {                   // empty context: the output row is zero
      for (int i = threadIdx.x; i < G * D; i += kWaves * 64)
        static_cast<uint16_t*>(p.out)[b * p.o_sb + (int64_t)(h0 + i / D) * p.o_sh + i % D] = 0;
    }
    return;
  }
  const int t_begin = part * p.partition_size;
  const int t_end = min(ctx, t_begin + p.partition_size);
  const int nchunks = (t_end - t_begin + kChunk - 1) / kChunk;

  // The G query rows of this kv head, this lane's 8 elements.
  uint32_t qv[G][4];
  float qsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) +
                                                    b * p.q_sb + (int64_t)(h0 + g) * p.q_sh + c * 8);
    qv[g][0] = v.x; qv[g][1] = v.y; qv[g][2] = v.z; qv[g][3] = v.w;
    qsum[g] = 0.f;
    if constexpr (KIND == CacheKind::U3) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) s += h_lo<BF16>(qv[g][e]) + h_hi<BF16>(qv[g][e]);
      qsum[g] = group_sum<LPR>(s);
    }
  }

  // Physical block of each of this wave's chunks (lane k <-> k-th chunk of the wave).
  int bt_lane = 0;
  {
    const int ck = w + lane * kWaves;
    if (ck < nchunks) {
      const int e = p.block_tables[b * p.bt_sb + ((t_begin + ck * kChunk) >> p.log2_bs)];
      bt_lane = (int)min<int64_t>(max(e, 0), p.num_blocks - 1);   // out-of-range ids clamped
    }
  }

  float m[G], l[G], zc[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = neg_inf();
    l[g] = 0.f;
    zc[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  const int64_t head_off = (int64_t)kvh * p.c_sh;
  for (int k = 0, ck = w; ck < nchunks; ++k, ck += kWaves) {
    const int tok0 = t_begin + ck * kChunk;
    const int phys = __builtin_amdgcn_readlane(bt_lane, k);
    const int slot0 = (tok0 & (p.block_size - 1)) + r;       // this row's slot at i = 0
    const int64_t row0 = (int64_t)phys * p.c_sb + (int64_t)slot0 * p.c_ss + head_off;

    bool valid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) valid[i] = tok0 + i * RPI + r < t_end;

    float sc[NI][G];
    float vf[NI][8];                 // V values (Same) or codes (U3)
    float vs[NI], vz[NI];            // U3: V scale / zero of the row
    if constexpr (KIND == CacheKind::Same) {
      uint4 kr[NI], vr[NI];
      const uint16_t* kb = static_cast<const uint16_t*>(p.k_cache) + row0 + c * 8;
      const uint16_t* vb = static_cast<const uint16_t*>(p.v_cache) + row0 + c * 8;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        kr[i] = *reinterpret_cast<const uint4*>(kb + (int64_t)i * RPI * p.c_ss);
        vr[i] = *reinterpret_cast<const uint4*>(vb + (int64_t)i * RPI * p.c_ss);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) d = dot2<BF16>(qv[g][e], kw[e], d);
          d = group_sum<LPR>(d);
          sc[i][g] = valid[i] ? d * p.scale_log2 : neg_inf();
        }
        const uint32_t vw[4] = {valid[i] ? vr[i].x : 0u, valid[i] ? vr[i].y : 0u,
                                valid[i] ? vr[i].z : 0u, valid[i] ? vr[i].w : 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[i][2 * e] = h_lo<BF16>(vw[e]);
          vf[i][2 * e + 1] = h_hi<BF16>(vw[e]);
        }
      }
    } else {
      // 3-bit rows: D*3/32 words; lane c owns octet c = stream bits [24c, 24c + 24), which
      // start in word 3c/4 at bit 24c mod 32 and spill into the next word for c mod 4 in {1, 2}.
      constexpr int WPR = D * 3 / 32;
      const int wj = (3 * c) >> 2;
      const int sh = (24 * c) & 31;
      const bool two = ((c & 3) == 1) || ((c & 3) == 2);
      const uint32_t* kb = static_cast<const uint32_t*>(p.k_cache) + row0 + wj;
      const uint32_t* vb = static_cast<const uint32_t*>(p.v_cache) + row0 + wj;
      const int64_t mbase = ((int64_t)phys * p.block_size + slot0) * p.num_kv_heads + kvh;
      const uint32_t* km = static_cast<const uint32_t*>(p.k_meta) + mbase;
      const uint32_t* vm = static_cast<const uint32_t*>(p.v_meta) + mbase;
      uint32_t klo[NI], khi[NI], vlo[NI], vhi[NI], kmeta[NI], vmeta[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t ro = (int64_t)i * RPI * p.c_ss;
        klo[i] = kb[ro];
        khi[i] = two ? kb[ro + 1] : 0u;
        vlo[i] = vb[ro];
        vhi[i] = two ? vb[ro + 1] : 0u;
        const int64_t mo = (int64_t)i * RPI * p.num_kv_heads;
        kmeta[i] = km[mo];
        vmeta[i] = vm[mo];
      }
      (void)WPR;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t ko = __builtin_amdgcn_alignbit(khi[i], klo[i], sh) & 0xffffffu;
        const float ks = f16_lo(kmeta[i]), kz = f16_hi(kmeta[i]);
        // codes as packed 16-bit pairs; bf16 pairs carry a +128 offset that is removed below
        uint32_t cp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = (ko >> (6 * e)) & 7u, bb = (ko >> (6 * e + 3)) & 7u;
          if constexpr (BF16) {
            cp[e] = (a | (bb << 16)) | 0x43004300u;              // 128 + code
          } else {
            const uint32_t magic = (a | (bb << 16)) | 0x64006400u;  // 1024 + code
            const f16x2_t v = __builtin_bit_cast(f16x2_t, magic) - (f16x2_t){1024.0f16, 1024.0f16};
            cp[e] = __builtin_bit_cast(uint32_t, v);
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) d = dot2<BF16>(qv[g][e], cp[e], d);
          d = group_sum<LPR>(d);
          const float off = BF16 ? 128.f + kz : kz;
          sc[i][g] = valid[i] ? ks * (d - off * qsum[g]) * p.scale_log2 : neg_inf();
        }
        const uint32_t vo = __builtin_amdgcn_alignbit(vhi[i], vlo[i], sh) & 0xffffffu;
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[i][e] = (float)((vo >> (3 * e)) & 7u);
        vs[i] = valid[i] ? f16_lo(vmeta[i]) : 0.f;
        vz[i] = valid[i] ? f16_hi(vmeta[i]) : 0.f;
      }
    }

    // online softmax update of each row's state
    float pp[NI][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = sc[0][g];
#pragma unroll
      for (int i = 1; i < NI; ++i) mx = fmaxf(mx, sc[i][g]);
      const float mn = fmaxf(m[g], mx);
      const float mu = (mn == neg_inf()) ? 0.f : mn;
      const float al = fast_exp2(m[g] - mu);
      m[g] = mn;
      l[g] *= al;
      zc[g] *= al;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= al;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        pp[i][g] = fast_exp2(sc[i][g] - mu);
        l[g] += pp[i][g];
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float pw = pp[i][g];
        if constexpr (KIND == CacheKind::U3) {
          pw *= vs[i];
          zc[g] = fmaf(pw, vz[i], zc[g]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pw, vf[i][e], acc[g][e]);
      }
    }
  }

  if constexpr (KIND == CacheKind::U3) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] -= zc[g];
  }

  // merge the token rows of this wave (lanes c, c + LPR, c + 2*LPR, ...)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      float mn, fs, fo;
      lse_factors(m[g], mo, mn, fs, fo);
      l[g] = l[g] * fs + lo * fo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[g][e], off);
        acc[g][e] = acc[g][e] * fs + ao * fo;
      }
      m[g] = mn;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[w][g][c * 8 + e] = acc[g][e];
      if (c == 0) {
        sm_m[w][g] = m[g];
        sm_l[w][g] = l[g];
      }
    }
  }
  __syncthreads();

  // merge the waves; write the output (single partition) or this partition's state
  for (int i = threadIdx.x; i < G * D; i += kWaves * 64) {
    const int g = i / D, d = i % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww][g]);
    const float mu = (M == neg_inf()) ? 0.f : M;
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(sm_m[ww][g] - mu);
      L += sm_l[ww][g] * f;
      A += sm_acc[ww][g][d] * f;
    }
    const int h = h0 + g;
    if (nparts == 1) {
      const float o = A / L;
      static_cast<uint16_t*>(p.out)[b * p.o_sb + (int64_t)h * p.o_sh + d] =
          (uint16_t)(BF16 ? f32_to_bf16_bits(o) : f32_to_f16_bits(o));
    } else {
      const int64_t slot = ((int64_t)b * p.num_q_heads + h) * p.max_parts + part;
      p.ws_acc[slot * D + d] = A;
      if (d == 0) {
        p.ws_ml[slot * 2] = M;
        p.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// Log-sum-exp merge of the partitions of each (request, query head); one thread per
// output element.  Requests that fit in one partition were written by the decode kernel.
template <int D, bool BF16>
__global__ __launch_bounds__(D) void merge_kernel(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int ctx = min(max(p.context_lens[b], 0), p.max_context_len);
  const int nparts = (ctx + p.partition_size - 1) / p.partition_size;
  if (nparts <= 1) return;
  const int64_t base = ((int64_t)b * p.num_q_heads + h) * p.max_parts;
  float M = neg_inf();
  for (int i = 0; i < nparts; ++i) M = fmaxf(M, p.ws_ml[(base + i) * 2]);
  float L = 0.f, A = 0.f;
  for (int i = 0; i < nparts; ++i) {
    const float f = fast_exp2(p.ws_ml[(base + i) * 2] - M);
    L += p.ws_ml[(base + i) * 2 + 1] * f;
    A += p.ws_acc[(base + i) * D + d] * f;
  }
  const float o = A / L;
  static_cast<uint16_t*>(p.out)[b * p.o_sb + (int64_t)h * p.o_sh + d] =
      (uint16_t)(BF16 ? f32_to_bf16_bits(o) : f32_to_f16_bits(o));
}

template <int D, int G, bool BF16, CacheKind KIND>
static hipError_t launch_t(const DecodeParams& p, int batch, hipStream_t s) {
  const int64_t wgs = (int64_t)p.max_parts * p.num_kv_heads * batch;
  hipLaunchKernelGGL((decode_kernel<D, G, BF16, KIND>), dim3((unsigned)wgs), dim3(kWaves * 64), 0, s,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_parts <= 1) return e;
  hipLaunchKernelGGL((merge_kernel<D, BF16>), dim3((unsigned)p.num_q_heads, (unsigned)batch),
                     dim3(D), 0, s, p);
  return hipGetLastError();
}

template <int D, int G, bool BF16>
static hipError_t by_kind(const DecodeParams& p, CacheKind kind, int batch, hipStream_t s) {
  if (kind == CacheKind::U3) return launch_t<D, G, BF16, CacheKind::U3>(p, batch, s);
  return launch_t<D, G, BF16, CacheKind::Same>(p, batch, s);
}

template <int D, bool BF16>
static hipError_t by_group(const DecodeParams& p, CacheKind kind, int group, int batch,
                           hipStream_t s) {
  switch (group) {
    case 1: return by_kind<D, 1, BF16>(p, kind, batch, s);
    case 2: return by_kind<D, 2, BF16>(p, kind, batch, s);
    case 4: return by_kind<D, 4, BF16>(p, kind, batch, s);
    case 8: return by_kind<D, 8, BF16>(p, kind, batch, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, CacheKind kind, bool bf16, int head_dim, int group,
                         int batch, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (head_dim == 128)
    return bf16 ? by_group<128, true>(p, kind, group, batch, s)
                : by_group<128, false>(p, kind, group, batch, s);
  return bf16 ? by_group<64, true>(p, kind, group, batch, s)
              : by_group<64, false>(p, kind, group, batch, s);
}

int auto_partition_size(int max_context_len, int batch, int num_q_heads) {
  (void)max_context_len;
  (void)batch;
  (void)num_q_heads;
  return 512;
}

}  // namespace pkv

// Paged decode attention (one query token per request), balanced split-K.
//
// What is computed ("Triton KV Cache and PagedAttention", Step 1 and the reference
// answer, TODO 1-5): for request b and query head h, out = sum_t softmax_t(sm_scale *
// q.k_t) v_t over the first context_lens[b] tokens; token t lives in physical block
// block_tables[b, t / block_size] at slot t % block_size; tokens past the context are
// masked; the softmax is accumulated online (running max m, running sum l, unnormalised
// accumulator).  GQA ("Write Triton Kv Cache Append Kernel", Kernel design rules): the G =
// Hq / Hkv query heads h = kvh*G .. kvh*G+G-1 share kv head kvh.  The 3-bit cache
// ("triton-3bit-kv-cache-kernel" README, title paragraph and section 2) is unpacked and
// dequantised, x = (q - z) * s, in registers; the byte-code caches (fp8 e4m3fn, fp8 e5m2,
// int8) read as decode(code) * s with the row's scale (the inverse of the append's quantiser,
// "Write Triton Kv Cache Append Kernel", Inputs item 4 and Correctness requirements).  Split-K: the context of a (request, kv head)
// may be cut at multiples of the partition size into ranges that are reduced separately
// and merged by log-sum-exp (the flash-decoding form the 3-bit README names).
//
// MI355X mapping:
//  * Memory: one slot of a block stores all kv heads of a token contiguously
//    ([block, slot, head, d]).  A wave instruction reads HPI heads x D elements of one
//    token (1 KB for 4 heads of 128 bf16), and the waves of a workgroup cover the other
//    heads of the same tokens at the same time, so whole slot rows are streamed and each
//    opened DRAM page is used in full.  Lane layout: D/8 lanes per (head, token) row, each
//    lane owning 8 consecutive elements (one 16-byte load of K and one of V; 8 bytes of
//    codes for the byte-code caches).  The K/V stream is loaded with the non-temporal hint: it is read once.
//  * Work (stream-K): requests are cut into granules of `partition_size` tokens; the
//    (request, head group, granule) units are laid end to end and the grid holds as many
//    workgroups as the chip keeps resident, each taking a contiguous range of units sized
//    to its expected speed, so that all workgroups stream for about the same time.  A
//    (request, head group) segment covered by one workgroup is finished in registers; where
//    a range starts or ends inside a segment the partial state (m, l, acc) goes to the
//    workspace and a small second kernel merges it by log-sum-exp.  Inside a workgroup the
//    waves are head waves (HPI heads each) times token streams (up to 4): the token streams
//    of a head wave share its chunks out through an LDS counter and merge their states
//    through LDS at the end of each segment.
//  * QK: where a wave instruction holds one token of HPI heads (the matrix-core form), the
//    scores of a chunk are v_mfma_f32_4x4x4 products with K token-transposed (a quad's lanes
//    hold 4 tokens) and the q heads as columns, summed over the quads of a row by DPP; else
//    v_dot2_f32_{bf16,f16} on packed pairs and a DPP reduction inside the lane row.  Each
//    lane keeps the online-softmax state of its own query heads (m, l in log2 units, the
//    lane's 8 accumulator columns per query head).
//  * Physical block ids of up to 64 blocks are fetched with one vector load (lane j <->
//    j-th block) and read back with v_readlane; the K/V loads of the next chunks are issued
//    before the current chunk is computed (a ring of register buffers).
#pragma once
#include <algorithm>
#include <type_traits>

#include "launch.h"
#include "common.cuh"
#include "fp8_quant.cuh"
#include "append_rows.cuh"

namespace pkv {

#ifndef PKV_PREFETCH_DEPTH
#define PKV_PREFETCH_DEPTH 2
#endif

constexpr int kMaxWaves = 8;        // waves per workgroup at most (token streams x head group)

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ int clamp_ctx(const DecodeParams& p, int b) {
  return min(max(p.context_lens[b], 0), p.max_context_len);
}

// Static split of the units over the grid.  Workgroup w carries a share proportional to a
// weight that depends on its dispatch tier and on the parity of w: the first workgroup
// dispatched to each CU (w < split_tier) is issued ahead of the CU's later ones and streams
// faster, and workgroups run on XCD w mod 8, where the odd-numbered XCDs were measured to
// stream more slowly.  Workgroup w starts at unit floor(total * c(w) / c(W)), c(w) = the sum
// of the weights of workgroups 0 .. w-1.
__device__ __forceinline__ int64_t split_c(const DecodeParams& p, int64_t w) {
  auto part = [&](int64_t n0, int64_t n1, int tier) {     // weights of workgroups [n0, n1)
    const int64_t evens = (n1 + 1) / 2 - (n0 + 1) / 2, odds = n1 / 2 - n0 / 2;
    return evens * p.split_w[2 * tier] + odds * p.split_w[2 * tier + 1];
  };
  const int64_t h = p.split_tier;
  return w <= h ? part(0, w, 0) : part(0, h, 0) + part(h, w, 1);
}
__device__ __forceinline__ int64_t range_start(const DecodeParams& p, int64_t total, int64_t w) {
  return total * split_c(p, w) / split_c(p, p.num_wgs);
}

// Lane geometry for head_dim D with HPI heads per wave instruction (G query heads per kv head).
template <int D, int HPI, int G>
struct Geo {
  static constexpr int LPR = D / 8;                 // lanes per (head, token) row
  static constexpr int RPI = 64 / LPR;              // rows per wave instruction
  static constexpr int TPI = RPI / HPI;             // tokens per wave instruction
  static constexpr int NI = (16 / TPI) < 4 ? (16 / TPI) : 4;   // instructions per chunk
  static constexpr int CT = NI * TPI;               // tokens per chunk (divides 16)
  static_assert(RPI % HPI == 0 && 16 % CT == 0, "lane geometry");
};

// byte-code caches (fp8 e4m3fn, fp8 e5m2, int8)
// codes in bytes 2 HI and 2 HI + 1 of w -> a packed pair of 16-bit values, or two fp32 values
template <CacheKind KIND, bool BF16, bool HI>
__device__ __forceinline__ uint32_t codes2_to_16(uint32_t w) {
  if constexpr (KIND == CacheKind::Fp8) return fp8x2_to_16<BF16, HI>(w);
  else if constexpr (KIND == CacheKind::E5m2) return e5m2x2_to_16<BF16, HI>(w);
  else return i8x2_to_16<BF16, HI>(w);
}
template <CacheKind KIND, bool HI>
__device__ __forceinline__ void codes2_to_f32(uint32_t w, float& lo, float& hi) {
  if constexpr (KIND == CacheKind::Fp8) fp8x2_to_f32<HI>(w, lo, hi);
  else if constexpr (KIND == CacheKind::E5m2) e5m2x2_to_f32<HI>(w, lo, hi);
  else i8x2_to_f32<HI>(w, lo, hi);
}

template <int NI, CacheKind KIND> struct Regs {
  uint2 k[NI], v[NI];                // 8 codes of the lane's row
  float ks[NI], vs[NI];              // the row's scales
};
template <int NI> struct Regs<NI, CacheKind::Same> { uint4 k[NI], v[NI]; };
template <int NI> struct Regs<NI, CacheKind::U3> {
  uint32_t klo[NI], khi[NI], vlo[NI], vhi[NI], km[NI], vm[NI];
};

template <int G>
struct State {
  uint32_t qv[G][4];                 // this lane's 8 query elements of each query head
  // matrix-core score form: the lane's query elements (8 per load instruction of a chunk) of the
  // query heads of its column (head q, and q + 4 with 8 heads), as the B operands
  uint32_t qm[G == 8 ? 2 : 1][4][4];
  float qsum[G];                     // u3: sum of the query row (dequant hoisting)
  float m[G], l[G], zc[G];
  // own-head form (see own_head_form): this lane's query head's running max, sum, zero-point
  // term and query sum; m, l and zc above hold every head's values again from range end on
  float mo[2], lo[2], zco[2], qso[2];
  // accumulator column e (this lane's d = 8c + e) of query head g is acc4[g / 4][e][g % 4]: the
  // register quads are the C operands of the PV matrix-core products
  f32x4_t acc4[(G + 3) / 4][8];
};

#define PKV_ACC(S, g, e) ((S).acc4[(g) >> 2][e][(g) & 3])

// acc[g][e] += w * p[g] * v[e] for the query heads g of this lane's row.  On the matrix cores:
// v_mfma_f32_4x4x1f32 runs 16 independent 4x4 outer products per wave, block b taking
// A[m] from lane 4b + m and B[n] from lane 4b + n and leaving C[m][n] in register m of lane
// 4b + n.  The 4 lanes of a block lie in one (head, token) row (D/8 lanes, a multiple of 4),
// all of which hold the row's p[g]; so with A = w * p[lane % 4] and B = v[e] of the lane
// itself, register m of lane (row, c) gains w * p[m] * v[e], the same as the FMA form.
// With G = 8 the extra operand registers push the kernel into spills (measured 7 % slower on
// the long-context decode), so G = 8 keeps the FMA form.
constexpr int kMfmaMaxG = 4;

// Own-head form (2, 4 or 8 query heads per kv head): after the score products a reduce-scatter
// over the quad (two DPP stages that halve the head set) and a sum over the quads of the row
// (two rotations for 16-lane rows, one lane permute for 8-lane rows) leave in lane q of every
// quad the full score of query head q mod G (heads q and q + 4 with G = 8), instead of every
// head's score in every lane.  The online softmax then runs for the lane's own heads only (a
// quarter of the exponentials), the matrix-core PV takes its A operand straight from the lane,
// and the per-head running sums are gathered back into every lane once, at the end of the
// lane's ranges.  The running maxima stay replicated (one quad broadcast per chunk), since every
// lane rescales the accumulators of all heads.  Measured against the replicated form: Llama-8B
// step 0.675 -> 0.690 of the HBM peak, fp8 decode 0.434 -> 0.488, 3-bit decode 0.167 -> 0.193,
// long context (8 heads) 0.607 -> 0.653; head_dim 64, 4 / 8 heads: 0.580 -> 0.593, 0.42 -> 0.44.
template <int D, int G> constexpr bool own_head_form() { return G == 2 || G == 4 || G == 8; }
// heads a lane owns: q mod G (G <= 4), or q and q + 4 (G = 8)
template <int G> constexpr int own_heads() { return G == 8 ? 2 : 1; }

// Matrix-core score form (own-head groups whose wave instruction holds one token of HPI heads,
// i.e. HPI = 64 / (D / 8)).  The score products of a chunk's 4 tokens are 4x4x4 matrix-core
// blocks: each quad of lanes is a block whose A operand is K (row m = token m of the chunk, the
// lane's 4 head-dim elements of it) and whose B operand is q (column n = query head n, the same
// 4 elements), so register m of lane n of the quad gains the partial score of token m for
// query head n - the own-head layout (lane q holds head q) with the chunk's tokens in its
// registers.  To feed it, the K loads are token-transposed: lane n of every quad reads token n,
// and the chunk's 4 load instructions walk 4 slices of the head dim (lane of quad cq of a row,
// instruction i: elements 8 j .. 8 j + 7 with j = mq_slice(i, cq)).  The quads of a row hold
// partial sums over disjoint slices and are summed once per chunk.  V keeps the row-major
// mapping (instruction i = token i).  With 8 query heads per kv head a second block set takes
// heads 4 .. 7; with 2, columns 2 and 3 repeat heads 0 and 1.  This replaces the 4 G dot2 products
// and the quad reduce-scatter of every token row with 2 own_heads matrix-core instructions per
// load instruction and one row sum per chunk.
template <int D, int G, int HPI>
constexpr bool mq_form() { return own_head_form<D, G>() && Geo<D, HPI, G>::TPI == 1; }
// The head-dim slice (8 elements) that instruction i of a chunk gives the lane of quad cq of a
// row in the matrix-core form: i * (LPR / 4) + cq for 16-bit caches.  The coded caches pair the
// slices instead (slices 2 j and 2 j + 1, j = (i / 2) * (LPR / 4) + cq, for instructions i and
// i + 1), so that one K load feeds two instructions: byte codes one 16-byte load instead of two
// 8-byte ones (the byte-code decodes are bound by their load stream: a loads-only copy of the
// kernel is as slow as the full one), 3-bit codes one 8-byte load instead of four 4-byte ones
// (the 6 bytes of two octets always lie in two aligned words).
template <int LPR, CacheKind KIND>
__device__ __forceinline__ constexpr int mq_slice(int i, int cq) {
  return KIND != CacheKind::Same ? 2 * ((i >> 1) * (LPR / 4) + cq) + (i & 1) : i * (LPR / 4) + cq;
}
// 3-bit codes, matrix-core form: the byte permute that lines octet j up from the 8 bytes of the
// word pair holding octets j & ~1 and (j & ~1) + 1 (they start at byte (3 (j & ~1)) mod 4, which
// is 0 or 2, and octet j + 1 three bytes later), arranged for the packed 16-bit shifts (bytes
// o, o + 1 in the low half, o + 1, o + 2 in the high half)
__device__ __forceinline__ uint32_t u3_pair_sel(int j) {
  const uint32_t o = (uint32_t)((3 * (j & ~1)) & 3) + 3u * (uint32_t)(j & 1);
  return o * 0x01010101u + 0x02010100u;
}

// Chunks whose loads are in flight at once per wave in the static-split loop (register buffers,
// one being computed).  The 16-bit caches move 8 KB per wave per chunk and saturate the memory
// path with two buffers (a third measured 1.5 % slower).  The byte-code and 3-bit caches move
// 2.1 KB and 1.7 KB; with 8-byte K loads (4 per chunk) they were faster with three buffers, and
// with the paired K loads (mq_slice: 2 per chunk) two are faster again (fp8 decode 0.534 -> 0.544
// of 8 TB/s, 3-bit decode 0.263 -> 0.272, 28 and 20 fewer VGPRs; four: slower).
template <int D, int G, CacheKind KIND, int HPI>
constexpr int prefetch_depth() {
  if constexpr (KIND == CacheKind::Same || !mq_form<D, G, HPI>() || G == 8) return 2;
  else return PKV_PREFETCH_DEPTH;
}

// The full scores of the lane's own heads from its partial dot products d[g], for rows of LPR
// lanes (16: D = 128; 8: D = 64).
template <int G, int LPR>
__device__ __forceinline__ void reduce_own(const float (&d)[G], int q, float (&s)[own_heads<G>()]) {
  const bool b0 = (q & 1) != 0, b1 = (q & 2) != 0;
  if constexpr (G == 8) {
    // keep the heads whose bit 0 is the lane's (head 2j + b0), add the partner's copy of them
    float k[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      k[j] = (b0 ? d[2 * j + 1] : d[2 * j]) + dpp_f<DPP_QUAD_XOR1>(b0 ? d[2 * j] : d[2 * j + 1]);
    // keep the heads whose bit 1 is the lane's: q and q + 4
    s[0] = (b1 ? k[1] : k[0]) + dpp_f<DPP_QUAD_XOR2>(b1 ? k[0] : k[1]);
    s[1] = (b1 ? k[3] : k[2]) + dpp_f<DPP_QUAD_XOR2>(b1 ? k[2] : k[3]);
  } else if constexpr (G == 4) {
    // keep the heads whose bit 0 is the lane's, add the partner's copy of them
    const float k0 = (b0 ? d[1] : d[0]) + dpp_f<DPP_QUAD_XOR1>(b0 ? d[0] : d[1]);
    const float k1 = (b0 ? d[3] : d[2]) + dpp_f<DPP_QUAD_XOR1>(b0 ? d[2] : d[3]);
    // keep the head whose bit 1 is the lane's
    s[0] = (b1 ? k1 : k0) + dpp_f<DPP_QUAD_XOR2>(b1 ? k0 : k1);
  } else {
    s[0] = (b0 ? d[1] : d[0]) + dpp_f<DPP_QUAD_XOR1>(b0 ? d[0] : d[1]);
    s[0] += dpp_f<DPP_QUAD_XOR2>(s[0]);
  }
  if constexpr (LPR == 16) {
    // the four quads of the row: rotations by 8 and then 4 keep a lane's place in its quad.  In
    // this order every quad adds the same pairs, (s0 + s2) + (s1 + s3) up to the order of the
    // operands of each addition, so all four quads hold bit-identical scores, and the row's
    // running maxima and sums (taken from its first quad where one value per row is written)
    // are those its accumulators were built with.  (Rotating by 4 first pairs the quads
    // differently in different quads.)
#pragma unroll
    for (int h = 0; h < own_heads<G>(); ++h) s[h] += dpp_f<DPP_ROW_ROR8>(s[h]);
#pragma unroll
    for (int h = 0; h < own_heads<G>(); ++h) s[h] += dpp_f<DPP_ROW_ROR4>(s[h]);
  } else {
    // the two quads of an 8-lane row: lane i and lane i ^ 4 (a cross-lane permute)
#pragma unroll
    for (int h = 0; h < own_heads<G>(); ++h) s[h] += __shfl_xor(s[h], 4);
  }
}

// every head's value from the lanes that own it: out[g] = x[h] of lane g % 4 of the quad for
// the own-head slot h = g / 4
template <int G>
__device__ __forceinline__ void quad_gather(const float* x, float (&out)[G]) {
#pragma unroll
  for (int h = 0; h < own_heads<G>(); ++h) {
    out[4 * h] = dpp_f<dpp_quad_bcast<0>()>(x[h]);
    if constexpr (G > 1) out[4 * h + 1] = dpp_f<dpp_quad_bcast<1>()>(x[h]);
    if constexpr (G > 2) out[4 * h + 2] = dpp_f<dpp_quad_bcast<2>()>(x[h]);
    if constexpr (G > 3) out[4 * h + 3] = dpp_f<dpp_quad_bcast<3>()>(x[h]);
  }
}

// x of lane i of the lane's quad (i known once the loops are unrolled)
__device__ __forceinline__ uint32_t quad_lane(uint32_t x, int i) {
  switch (i) {
    case 0: return dpp_u<dpp_quad_bcast<0>()>(x);
    case 1: return dpp_u<dpp_quad_bcast<1>()>(x);
    case 2: return dpp_u<dpp_quad_bcast<2>()>(x);
    default: return dpp_u<dpp_quad_bcast<3>()>(x);
  }
}

template <int G, typename St>
__device__ __forceinline__ void pv_accumulate(St& S, const float (&p)[G], float w, const float (&v)[8]) {
  if constexpr (G <= kMfmaMaxG) {
    const int q = threadIdx.x & 3;
#pragma unroll
    for (int h4 = 0; h4 < (G + 3) / 4; ++h4) {      // query heads 4 h4 .. 4 h4 + 3
      float a = 0.f;                                // heads g >= G of the quad stay 0
#pragma unroll
      for (int m = 0; m < 4 && 4 * h4 + m < G; ++m) a = (q == m) ? p[4 * h4 + m] : a;
      a *= w;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        S.acc4[h4][e] = __builtin_amdgcn_mfma_f32_4x4x1f32(a, v[e], S.acc4[h4][e], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pw = p[g] * w;
#pragma unroll
      for (int e = 0; e < 8; ++e) PKV_ACC(S, g, e) = fmaf(pw, v[e], PKV_ACC(S, g, e));
    }
  }
}

// The own-head form of pv_accumulate: po is this lane's head's probability, which is the A
// operand lane q % 4 of each block supplies (query heads >= G contribute 0).
// With 8 heads the matrix-core form spills, so the probabilities are gathered into every lane
// (two quad broadcasts per head set) and the FMA form of pv_accumulate is kept.
template <int G, typename St>
__device__ __forceinline__ void pv_accumulate_own(St& S, const float (&po)[own_heads<G>()], float w,
                                                  const float (&v)[8], int q) {
  if constexpr (G <= kMfmaMaxG) {
    const float a = (G == 4 || q < G) ? po[0] * w : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) S.acc4[0][e] = __builtin_amdgcn_mfma_f32_4x4x1f32(a, v[e], S.acc4[0][e], 0, 0, 0);
  } else {
    float pg[G];
    quad_gather<G>(po, pg);
    pv_accumulate<G>(S, pg, w, v);
  }
}

// Per-lane byte offsets of the rows a lane reads in a chunk (instruction i reads the row
// TPI*i slots after the lane's first row); the chunk's block and first slot are
// wave-uniform and kept in scalar registers.
template <int D, int HPI, CacheKind KIND, int G>
struct LaneOffsets {
  static constexpr int NI = Geo<D, HPI, G>::NI;
  uint32_t row[NI];                  // bytes from the chunk's uniform row base
  uint32_t meta[NI];                 // u3: bytes from the chunk's uniform meta base
  // matrix-core score form: the K rows of load instruction i (token-transposed; the coded
  // caches load at even i the slices of instructions i and i + 1; 3-bit: the first of the two
  // words that hold the lane's octet pair); V and meta of token 0 (token i adds i slot strides)
  uint32_t krow[NI];
  uint32_t vrow, vrow_hi;
  uint32_t mrow;                     // meta of token (lane mod 4) of the chunk, the lane's head
};

template <int D, int HPI, CacheKind KIND, int G>
__device__ __forceinline__ LaneOffsets<D, HPI, KIND, G> lane_offsets(const DecodeParams& p, int tr, int hh,
                                                                   int c) {
  using Gm = Geo<D, HPI, G>;
  LaneOffsets<D, HPI, KIND, G> o;
  constexpr int esz = KIND == CacheKind::U3 ? 4 : byte_kind(KIND) ? 1 : 2;
  const int col = KIND == CacheKind::U3 ? ((3 * c) >> 2) : c * 8;
#pragma unroll
  for (int i = 0; i < Gm::NI; ++i) {
    const int64_t slot = tr + i * Gm::TPI;
    o.row[i] = (uint32_t)((slot * p.c_ss + (int64_t)hh * p.c_sh + col) * esz);
    o.meta[i] = (uint32_t)((slot * p.m_ss + (int64_t)hh * p.m_sh) * 4);
  }
  if constexpr (mq_form<D, G, HPI>()) {
    const int n = c & 3, cq = c >> 2;
    const int64_t krow0 = (int64_t)n * p.c_ss + (int64_t)hh * p.c_sh;
#pragma unroll
    for (int i = 0; i < Gm::NI; ++i) {
      const int j = mq_slice<Gm::LPR, KIND>(i, cq);    // the lane's 8-element slice of the head dim
      if constexpr (KIND == CacheKind::U3) {
        // octet j = stream bits [24 j, 24 j + 24): octets j & ~1 and its successor fill bytes
        // [3 (j & ~1), 3 (j & ~1) + 6), inside words 3 (j & ~1) / 4 and the next one
        o.krow[i] = (uint32_t)((krow0 + ((3 * (j & ~1)) >> 2)) * 4);
      } else {
        o.krow[i] = (uint32_t)((krow0 + 8 * j) * esz);
      }
    }
    const bool vtwo = ((c & 3) == 1) || ((c & 3) == 2);
    o.vrow = (uint32_t)(((int64_t)hh * p.c_sh + col) * esz);
    o.vrow_hi = o.vrow + ((KIND == CacheKind::U3 && vtwo) ? 4u : 0u);
    o.mrow = (uint32_t)(((int64_t)n * p.m_ss + (int64_t)hh * p.m_sh) * 4);   // token n's meta
  }
  return o;
}

// Issue the loads of one chunk: `kb`/`vb` point at the row of (block, first slot, first head
// of the group) and `kmb`/`vmb` at its meta entry (u3), all wave-uniform.
template <int D, int HPI, CacheKind KIND, int G>
__device__ __forceinline__ void load_chunk(const DecodeParams& p, const char* kb, const char* vb,
                                           const char* kmb, const char* vmb,
                                           const LaneOffsets<D, HPI, KIND, G>& o, int c,
                                           Regs<Geo<D, HPI, G>::NI, KIND>& R, bool live = true) {
  using Gm = Geo<D, HPI, G>;
  if constexpr (mq_form<D, G, HPI>()) {
    // a chunk that is not live (past the end of the range) is loaded through resources of 0
    // records: zeros, no memory access, the same instructions
    const int nrec = live ? 0x7fffffff : 0;
    // buffer loads: K token-transposed (instruction i = a head-dim slice of the chunk's 4
    // tokens), V and meta row-major (instruction i = token i, i slot strides further on).  The K
    // loads carry no non-temporal hint: each K instruction reads part of 16 cache lines that the
    // chunk's other 3 K instructions read too, so the lines must stay in the vector cache until
    // then (with the hint: fp8 decode 74.6 -> 83.1 us, 3-bit decode 131.5 -> 144.2 us on one box).
    // V, read in whole lines by each instruction, keeps it.
    constexpr int esz = KIND == CacheKind::U3 ? 4 : byte_kind(KIND) ? 1 : 2;
    const uint32_t ss = (uint32_t)(p.c_ss * esz);
    const BufRsrc kr = buf_rsrc(kb, nrec), vr = buf_rsrc(vb, nrec);
    if constexpr (KIND == CacheKind::Same) {
#pragma unroll
      for (int i = 0; i < Gm::NI; ++i) {
        R.k[i] = buf_load_u4<false>(kr, o.krow[i], 0);
        R.v[i] = buf_load_u4<true>(vr, o.vrow, i * ss);
      }
    } else if constexpr (byte_kind(KIND)) {
      // the chunk's 4 row scales of the lane's head in one load each for K and V: lane q of a
      // quad reads token q's (slot 0 of the registers; spread over the quad when computed)
      const BufRsrc kmr = buf_rsrc(kmb, nrec), vmr = buf_rsrc(vmb, nrec);
      R.ks[0] = __uint_as_float(buf_load_u32<false>(kmr, o.mrow, 0));
      R.vs[0] = __uint_as_float(buf_load_u32<false>(vmr, o.mrow, 0));
      static_assert(Gm::NI % 2 == 0, "paired K slices");
#pragma unroll
      for (int i = 0; i < Gm::NI; i += 2) {            // slices of instructions i, i + 1: one load
        const uint4 k2 = buf_load_u4<false>(kr, o.krow[i], 0);
        R.k[i] = make_uint2(k2.x, k2.y);
        R.k[i + 1] = make_uint2(k2.z, k2.w);
      }
#pragma unroll
      for (int i = 0; i < Gm::NI; ++i) R.v[i] = buf_load_u2<true>(vr, o.vrow, i * ss);
    } else {
      const BufRsrc kmr = buf_rsrc(kmb, nrec), vmr = buf_rsrc(vmb, nrec);
      R.km[0] = buf_load_u32<true>(kmr, o.mrow, 0);          // (s, z) of token lane mod 4
      R.vm[0] = buf_load_u32<true>(vmr, o.mrow, 0);
#pragma unroll
      for (int i = 0; i < Gm::NI; i += 2) {            // octets of instructions i, i + 1: one load
        const uint2 kw = buf_load_u2<false>(kr, o.krow[i], 0);
        R.klo[i] = R.klo[i + 1] = kw.x;
        R.khi[i] = R.khi[i + 1] = kw.y;
      }
#pragma unroll
      for (int i = 0; i < Gm::NI; ++i) {
        R.vlo[i] = buf_load_u32<true>(vr, o.vrow, i * ss);
        R.vhi[i] = buf_load_u32<true>(vr, o.vrow_hi, i * ss);
      }
    }
    return;
  }
  if constexpr (KIND == CacheKind::Same) {
#pragma unroll
    for (int i = 0; i < Gm::NI; ++i) {
      R.k[i] = load_stream_u4(kb + o.row[i]);
      R.v[i] = load_stream_u4(vb + o.row[i]);
    }
  } else if constexpr (byte_kind(KIND)) {
#pragma unroll
    for (int i = 0; i < Gm::NI; ++i) {
      R.k[i] = load_stream_u2(kb + o.row[i]);
      R.v[i] = load_stream_u2(vb + o.row[i]);
      R.ks[i] = *reinterpret_cast<const float*>(kmb + o.meta[i]);
      R.vs[i] = *reinterpret_cast<const float*>(vmb + o.meta[i]);
    }
  } else {
    // 3-bit rows: D*3/32 words; lane c owns octet c = stream bits [24c, 24c + 24), which
    // start in word 3c/4 and spill into the next word for c mod 4 in {1, 2}.
    const bool two = ((c & 3) == 1) || ((c & 3) == 2);
#pragma unroll
    for (int i = 0; i < Gm::NI; ++i) {
      R.klo[i] = load_stream_u32(kb + o.row[i]);
      R.khi[i] = two ? load_stream_u32(kb + o.row[i] + 4) : 0u;
      R.vlo[i] = load_stream_u32(vb + o.row[i]);
      R.vhi[i] = two ? load_stream_u32(vb + o.row[i] + 4) : 0u;
      R.km[i] = load_stream_u32(kmb + o.meta[i]);
      R.vm[i] = load_stream_u32(vmb + o.meta[i]);
    }
  }
}

// QK, online-softmax update and PV for one chunk of this lane's row.  MASKED: tokens at or
// past t_end are excluded (only the last chunk of a range can be ragged).
template <int D, int G, bool BF16, CacheKind KIND, int HPI, bool MASKED>
__device__ __forceinline__ void compute_chunk(const DecodeParams& p, State<G>& S,
                                              const Regs<Geo<D, HPI, G>::NI, KIND>& R, int tok,
                                              int t_end, int c) {
  using Gm = Geo<D, HPI, G>;
  constexpr int NI = Gm::NI, LPR = Gm::LPR;
  bool valid[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) valid[i] = !MASKED || (tok + i * Gm::TPI < t_end);
  constexpr bool OWN = own_head_form<D, G>();
  const int q = threadIdx.x & 3;
  float sc[NI][G];                   // every head's scores (OWN: unused)
  constexpr int HO = own_heads<G>();
  float sco[NI][HO];                 // OWN: this lane's heads' scores
  // the row meta of token i (byte codes: fp32 scales; 3-bit: fp16 (s, z)): in register i of the
  // row-major form; in the matrix-core score form lane q of each quad loaded token q's
  [[maybe_unused]] uint32_t kmt[NI], vmt[NI];
  if constexpr (byte_kind(KIND) || KIND == CacheKind::U3) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (byte_kind(KIND)) {
        kmt[i] = mq_form<D, G, HPI>() ? quad_lane(__float_as_uint(R.ks[0]), i) : __float_as_uint(R.ks[i]);
        vmt[i] = mq_form<D, G, HPI>() ? quad_lane(__float_as_uint(R.vs[0]), i) : __float_as_uint(R.vs[i]);
      } else {
        kmt[i] = mq_form<D, G, HPI>() ? quad_lane(R.km[0], i) : R.km[i];
        vmt[i] = mq_form<D, G, HPI>() ? quad_lane(R.vm[0], i) : R.vm[i];
      }
    }
  }
  if constexpr (mq_form<D, G, HPI>()) {
    // matrix-core score form: sacc[h] register i = token i's score for the lane's column head
    f32x4_t sacc[HO];
#pragma unroll
    for (int h = 0; h < HO; ++h) sacc[h] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // the lane's 8 K elements of slice i as four packed 16-bit pairs, in the element order of
      // the query pairs S.qm[.][i]
      uint32_t kw[4];
      if constexpr (KIND == CacheKind::Same) {
        kw[0] = R.k[i].x; kw[1] = R.k[i].y; kw[2] = R.k[i].z; kw[3] = R.k[i].w;
      } else if constexpr (byte_kind(KIND)) {
        kw[0] = codes2_to_16<KIND, BF16, false>(R.k[i].x);
        kw[1] = codes2_to_16<KIND, BF16, true>(R.k[i].x);
        kw[2] = codes2_to_16<KIND, BF16, false>(R.k[i].y);
        kw[3] = codes2_to_16<KIND, BF16, true>(R.k[i].y);
      } else {
        // octet j of the row from the word pair (klo, khi) that holds it: the permute and the
        // packed shifts of the row-major form, pairs (code e, code e + 4)
        const uint32_t y = __builtin_amdgcn_perm(R.khi[i], R.klo[i], u3_pair_sel(mq_slice<LPR, KIND>(i, c >> 2)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u16x2_t sh2 = {(uint16_t)(3 * e), (uint16_t)(3 * e + 4)};
          const uint32_t pr = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, y) >> sh2) & 0x00070007u;
          // bf16: 128 + code (exact; the 128 is folded into the zero point); fp16: the code alone
          // is the subnormal code * 2^-24, which the matrix cores multiply exactly (the 2^24 is
          // folded into the scale and the query sum)
          kw[e] = BF16 ? (pr | 0x43004300u) : pr;
        }
      }
#pragma unroll
      for (int h = 0; h < HO; ++h) {
        sacc[h] = mfma4x4x4<BF16>(kw[0], kw[1], S.qm[h][i][0], S.qm[h][i][1], sacc[h]);
        sacc[h] = mfma4x4x4<BF16>(kw[2], kw[3], S.qm[h][i][2], S.qm[h][i][3], sacc[h]);
      }
    }
    // the row's quads summed over their head-dim slices, bit-identically in every quad
#pragma unroll
    for (int h = 0; h < HO; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[h][r] = row_quads_sum<LPR>(sacc[h][r]);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (KIND == CacheKind::U3) {
        // q.(code - z)*s = s * (q.code - z * sum(q)); bf16 codes carry +128 (folded into z);
        // fp16: sacc is q.code * 2^-24 and S.qso the query sum * 2^-24
        const float kz = f16_hi(kmt[i]);
        const float off = BF16 ? 128.f + kz : kz;
        const float kscl = BF16 ? p.scale_log2 : p.scale_log2 * 0x1p24f;
        // the scale times the score factor in one mixed-precision fma on the stored fp16 scale,
        // then one product per head
        const float ks2 = fmaf(f16_lo(kmt[i]), kscl, 0.f);
#pragma unroll
        for (int h = 0; h < HO; ++h)
          sco[i][h] = valid[i] ? ks2 * (sacc[h][i] - off * S.qso[h]) : neg_inf();
      } else {
        float scl = p.scale_log2;
        if constexpr (byte_kind(KIND)) scl *= __uint_as_float(kmt[i]);
#pragma unroll
        for (int h = 0; h < HO; ++h) sco[i][h] = valid[i] ? sacc[h][i] * scl : neg_inf();
      }
    }
  } else if constexpr (KIND == CacheKind::Same || byte_kind(KIND)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint32_t kw[4];
      if constexpr (KIND == CacheKind::Same) {
        kw[0] = R.k[i].x; kw[1] = R.k[i].y; kw[2] = R.k[i].z; kw[3] = R.k[i].w;
      } else {
        // byte codes: the 8 codes as exact 16-bit pairs of the query's type; the row scale
        // multiplies the dot product: (s k) . q = s (k . q)
        kw[0] = codes2_to_16<KIND, BF16, false>(R.k[i].x);
        kw[1] = codes2_to_16<KIND, BF16, true>(R.k[i].x);
        kw[2] = codes2_to_16<KIND, BF16, false>(R.k[i].y);
        kw[3] = codes2_to_16<KIND, BF16, true>(R.k[i].y);
      }
      float d[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        d[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[g] = dot2<BF16>(S.qv[g][e], kw[e], d[g]);
      }
      float scl = p.scale_log2;
      if constexpr (byte_kind(KIND)) scl *= __uint_as_float(kmt[i]);
      if constexpr (OWN) {
        float so[HO];
        reduce_own<G, LPR>(d, q, so);
#pragma unroll
        for (int h = 0; h < HO; ++h) sco[i][h] = valid[i] ? so[h] * scl : neg_inf();
      } else {
        // stage-major across the query heads: no DPP read waits on the instruction before it
        // (with 8 heads: long-context decode +1 %)
        group_sum_n<LPR>(d);
#pragma unroll
        for (int g = 0; g < G; ++g) sc[i][g] = valid[i] ? d[g] * scl : neg_inf();
      }
    }
  } else {
    // The lane's octet starts at byte (3c) mod 4 of (klo, khi); one byte permute gives
    // y = [bits 0..15 | bits 8..23] of the octet, so that code e sits at bit 3e of the low half
    // and code e + 4 at bit 3e + 4 of the high half, and one packed 16-bit shift per pair
    // lines up (code e, code e + 4) for the dot product with (q[e], q[e + 4]).
    const uint32_t sel = (uint32_t)((3 * c) & 3) * 0x01010101u + 0x02010100u;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t y = __builtin_amdgcn_perm(R.khi[i], R.klo[i], sel);
      // codes as packed 16-bit pairs: fp16 exactly (1024 + c, minus 1024); bf16 pairs keep a
      // +128 offset that is folded into the zero point below
      uint32_t cp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u16x2_t sh2 = {(uint16_t)(3 * e), (uint16_t)(3 * e + 4)};
        const uint32_t pr = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, y) >> sh2) & 0x00070007u;
        if constexpr (BF16) {
          cp[e] = pr | 0x43004300u;
        } else {
          const f16x2_t v = __builtin_bit_cast(f16x2_t, pr | 0x64006400u) - (f16x2_t){1024.0f16, 1024.0f16};
          cp[e] = __builtin_bit_cast(uint32_t, v);
        }
      }
      float d[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        d[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[g] = dot2<BF16>(S.qv[g][e], cp[e], d[g]);
      }
      const float ks = f16_lo(kmt[i]), kz = f16_hi(kmt[i]);
      const float off = BF16 ? 128.f + kz : kz;
      if constexpr (OWN) {
        float so[HO];
        reduce_own<G, LPR>(d, q, so);
#pragma unroll
        for (int h = 0; h < HO; ++h)
          sco[i][h] = valid[i] ? ks * (so[h] - off * S.qso[h]) * p.scale_log2 : neg_inf();
      } else {
        if constexpr (G <= 4) {
          group_sum_n<LPR>(d);
        } else {
#pragma unroll
          for (int g = 0; g < G; ++g) d[g] = group_sum<LPR>(d[g]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          // q.(code - z)*s = s * (q.code - z * sum(q))
          sc[i][g] = valid[i] ? ks * (d[g] - off * S.qsum[g]) * p.scale_log2 : neg_inf();
        }
      }
    }
  }
  // Online-softmax update.  The running maxima rarely grow once a few dozen tokens have been
  // seen, so the rescaling of (l, acc) is skipped for the whole wave when no row's maximum
  // grew in this chunk: the factor would be exp2(0) = 1 exactly, so the result is the same.
  float pp[NI][G];                   // every head's probabilities (OWN: unused)
  float ppo[NI][HO];                 // OWN: this lane's heads' probabilities
  float mx[G];
  float mxo[HO];
  bool grow = false;
  if constexpr (OWN) {
    // every head is owned by a lane of every quad, whose own maximum equals the replicated one,
    // so comparing the own heads decides for the wave; the replicated maxima of every head are
    // gathered only when some grew
#pragma unroll
    for (int h = 0; h < HO; ++h) {
      mxo[h] = sco[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) mxo[h] = fmaxf(mxo[h], sco[i][h]);
      grow |= mxo[h] > S.mo[h];
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mx[g] = sc[0][g];
#pragma unroll
      for (int i = 1; i < NI; ++i) mx[g] = fmaxf(mx[g], sc[i][g]);
      grow |= mx[g] > S.m[g];
    }
  }
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    if constexpr (OWN) quad_gather<G>(mxo, mx);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mn = fmaxf(S.m[g], mx[g]);
      const float mu = (MASKED && mn == neg_inf()) ? 0.f : mn;   // a row with no token yet
      const float al = fast_exp2(S.m[g] - mu);
      S.m[g] = mn;
      if constexpr (!OWN) {
        S.l[g] *= al;
        if constexpr (KIND == CacheKind::U3) S.zc[g] *= al;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) PKV_ACC(S, g, e) *= al;
    }
    if constexpr (OWN) {
#pragma unroll
      for (int h = 0; h < HO; ++h) {
        const float mn = fmaxf(S.mo[h], mxo[h]);
        const float mu = (MASKED && mn == neg_inf()) ? 0.f : mn;
        const float al = fast_exp2(S.mo[h] - mu);
        S.mo[h] = mn;
        S.lo[h] *= al;
        if constexpr (KIND == CacheKind::U3) S.zco[h] *= al;
      }
    }
  }
  if constexpr (OWN) {
#pragma unroll
    for (int h = 0; h < HO; ++h) {
      const float mu = (MASKED && S.mo[h] == neg_inf()) ? 0.f : S.mo[h];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        ppo[i][h] = fast_exp2(sco[i][h] - mu);
        S.lo[h] += ppo[i][h];
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mu = (MASKED && S.m[g] == neg_inf()) ? 0.f : S.m[g];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        pp[i][g] = fast_exp2(sc[i][g] - mu);
        S.l[g] += pp[i][g];
      }
    }
  }
  if constexpr (KIND == CacheKind::U3 && OWN && G <= kMfmaMaxG && NI == 4) {
    // 3-bit V on the matrix cores at 16 bits: per element e of the lane's 8, v_mfma_f32_4x4x4f16
    // sums the chunk's 4 tokens (k = token i).  A: lane q of a quad gives its own head's weights
    // w_i = p_i s_i, as two fp16 parts with one product each (below; p <= 1 and s is an fp16
    // value, so w cannot overflow); B: lane n gives element e of the 4 tokens as the exact fp16
    // value 8 + code (bits 0x4800 | code << 7).  Register m of lane n then gains
    // sum_i w_i (8 + code_i) for head m, as the fp32 form's sum_i (p_i s_i) code_i plus
    // 8 sum_i w_i.  The zero-point sum takes the same weights, sum_i w_i (z_i + 8), so that
    // acc - zc = sum_i w_i (code_i - z_i) as before.  The 8 (not 1024 + code, whose fp16
    // bits need no shift) keeps the offset within 3 bits of the codes in the fp32 sums.
    const uint32_t sel = (uint32_t)((3 * c) & 3) * 0x01010101u + 0x02010100u;
    // Token pair j = (2j, 2j + 1): each token's octet lined up by one byte permute
    // (y = [octet bits 0..15 | octet bits 8..23]), then the two tokens' low halves and high
    // halves paired by one more permute each: L = [bits 0..15 of token 2j | of token 2j + 1],
    // H = [bits 8..23 of token 2j | of token 2j + 1].  Code e sits at bit 3e of each half of L and
    // code e + 4 at bit 3e + 4 of each half of H, so one 32-bit shift moves both tokens' code to
    // bits 7..9 of their halves (what a shift carries across the halves lands outside bits 7..9),
    // and one mask-and-bias instruction gives the fp16 pair (8 + code of token 2j, of token
    // 2j + 1): the B operand of element e (L) or e + 4 (H).
    uint32_t bl[2][4], bh[2][4];
    const uint32_t cmask = p.u3_code_mask;
    // the bias in a vector register: v_and_or_b32 reads at most one scalar operand here
    uint32_t vbias = p.u3_code_bias;
    asm volatile("v_mov_b32 %0, %1" : "=v"(vbias) : "s"(vbias));
    auto mask_bias = [&](uint32_t x) {
      uint32_t r;
      asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(cmask), "v"(vbias));
      return r;
    };
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t y0 = __builtin_amdgcn_perm(R.vhi[2 * j], R.vlo[2 * j], sel);
      const uint32_t y1 = __builtin_amdgcn_perm(R.vhi[2 * j + 1], R.vlo[2 * j + 1], sel);
      const uint32_t L = __builtin_amdgcn_perm(y1, y0, 0x05040100u);
      const uint32_t H = __builtin_amdgcn_perm(y1, y0, 0x07060302u);
      bl[j][0] = mask_bias(L << 7);
      bl[j][1] = mask_bias(L << 4);
      bl[j][2] = mask_bias(L << 1);
      bl[j][3] = mask_bias(L >> 2);
      bh[j][0] = mask_bias(H << 3);
      bh[j][1] = mask_bias(H);
      bh[j][2] = mask_bias(H >> 3);
      bh[j][3] = mask_bias(H >> 6);
    }
    // the weights of tokens (0, 1) and (2, 3) as fp16 pairs, each weight w split into its fp16
    // rounding and the fp16 rounding of the rest (w - hi is exact in fp32), so that the two
    // products together carry w to about 2^-24 relative, like the fp32 form: with a single fp16
    // weight an output that is a small difference of large values (V rows of both signs with a
    // large scale) could lose more than the decode's tolerance
    uint32_t wp[2], wq[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      _Float16 wh[2], wl[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int i = 2 * j + t;
        const float vs = valid[i] ? f16_lo(vmt[i]) : 0.f;
        const float vz = valid[i] ? f16_hi(vmt[i]) : 0.f;
        const float w = ppo[i][0] * vs;
        wh[t] = (_Float16)w;
        wl[t] = (_Float16)(w - (float)wh[t]);
        S.zco[0] = fmaf(w, vz + 8.f, S.zco[0]);
      }
      // heads q >= G of a 2-head group add nothing (their columns repeat heads 0 and 1)
      const bool live = G == 4 || q < G;
      wp[j] = live ? (uint32_t)__builtin_bit_cast(uint16_t, wh[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, wh[1]) << 16)
                   : 0u;
      wq[j] = live ? (uint32_t)__builtin_bit_cast(uint16_t, wl[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, wl[1]) << 16)
                   : 0u;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      S.acc4[0][e] = mfma4x4x4<false>(wp[0], wp[1], bl[0][e], bl[1][e], S.acc4[0][e]);
      S.acc4[0][e + 4] = mfma4x4x4<false>(wp[0], wp[1], bh[0][e], bh[1][e], S.acc4[0][e + 4]);
      S.acc4[0][e] = mfma4x4x4<false>(wq[0], wq[1], bl[0][e], bl[1][e], S.acc4[0][e]);
      S.acc4[0][e + 4] = mfma4x4x4<false>(wq[0], wq[1], bh[0][e], bh[1][e], S.acc4[0][e + 4]);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float vf[8];
    if constexpr (KIND == CacheKind::Same) {
      uint32_t vw[4] = {R.v[i].x, R.v[i].y, R.v[i].z, R.v[i].w};
      if (MASKED && !valid[i]) vw[0] = vw[1] = vw[2] = vw[3] = 0u;   // poisoned tails stay out
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = h_lo<BF16>(vw[e]);
        vf[2 * e + 1] = h_hi<BF16>(vw[e]);
      }
      if constexpr (OWN) pv_accumulate_own<G>(S, ppo[i], 1.f, vf, q);
      else pv_accumulate<G>(S, pp[i], 1.f, vf);
    } else if constexpr (byte_kind(KIND)) {
      uint32_t vw0 = R.v[i].x, vw1 = R.v[i].y;
      float vs = __uint_as_float(vmt[i]);
      if (MASKED && !valid[i]) { vw0 = vw1 = 0u; vs = 0.f; }          // poisoned tails stay out
      codes2_to_f32<KIND, false>(vw0, vf[0], vf[1]);
      codes2_to_f32<KIND, true>(vw0, vf[2], vf[3]);
      codes2_to_f32<KIND, false>(vw1, vf[4], vf[5]);
      codes2_to_f32<KIND, true>(vw1, vf[6], vf[7]);
      // sum_t p (s v_t) = sum_t (p s) v_t
      if constexpr (OWN) pv_accumulate_own<G>(S, ppo[i], vs, vf, q);
      else pv_accumulate<G>(S, pp[i], vs, vf);
    } else {
      // the same byte permute: codes 0..4 at bits 3e, codes 5..7 at bits 3e + 8
      const uint32_t y = __builtin_amdgcn_perm(R.vhi[i], R.vlo[i], (uint32_t)((3 * c) & 3) * 0x01010101u + 0x02010100u);
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] = (float)((y >> (e < 5 ? 3 * e : 3 * e + 8)) & 7u);
      const float vs = valid[i] ? f16_lo(vmt[i]) : 0.f;
      const float vz = valid[i] ? f16_hi(vmt[i]) : 0.f;
      // sum_t p (code - z) s = sum_t (p s) code - sum_t (p s) z
      if constexpr (OWN) {
#pragma unroll
        for (int h = 0; h < HO; ++h) S.zco[h] = fmaf(ppo[i][h] * vs, vz, S.zco[h]);
        pv_accumulate_own<G>(S, ppo[i], vs, vf, q);
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) S.zc[g] = fmaf(pp[i][g] * vs, vz, S.zc[g]);
        pv_accumulate<G>(S, pp[i], vs, vf);
      }
    }
  }
}

// A wave that stored appended rows: once its stores have completed (s_waitcnt 0, which also waits
// for its loads in flight), count it in `done` (LDS).
__device__ __forceinline__ void count_appended(int* done) {
  __builtin_amdgcn_s_waitcnt(0);
  if ((threadIdx.x & 63) == 0) {
    typedef __attribute__((address_space(3))) int LdsInt;
    __hip_atomic_fetch_add((LdsInt*)done, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}
// Wait until `done` (LDS) reaches `target`: the rows this workgroup appended (append_new_rows) are in memory.
__device__ __forceinline__ void wait_appended(int* done, int target) {
  typedef __attribute__((address_space(3))) int LdsInt;
  while (__hip_atomic_load((LdsInt*)done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
    __builtin_amdgcn_s_sleep(1);
}

// Reduce the chunks of tokens [t0, t1) of request b, head group hg into S (this lane's row:
// head hh of the group, token offset tr inside a wave instruction).  The token streams of one
// head wave take the chunks from a counter in LDS (`cnt`, zero at the start) rather than a
// fixed interleave, so that a wave that streams faster (the SIMD issues the oldest waves
// first) takes more chunks and the workgroup's waves finish the range together.  Physical
// block ids of up to 64 blocks are fetched with one vector load (lane j <-> j-th block of the
// window) and read back with v_readlane; the K/V loads of the next chunks are issued before the
// current chunk is computed (a ring of register buffers).  With a fused append (new_tok >= 0) the
// chunk holding the appended token is loaded only once the workgroup's stores of it are counted.
template <int D, int G, bool BF16, CacheKind KIND, int HPI>
__device__ __forceinline__ void run_range(const DecodeParams& p, State<G>& S, int b, int hg, int t0,
                                                 int t1, int lane, int tr, int hh, int c, int* cnt,
                                                 int new_tok = -1, int* app_done = nullptr, int app_target = 0,
                                                 bool app_mine = false) {
  using Gm = Geo<D, HPI, G>;
  using R = Regs<Gm::NI, KIND>;
  constexpr int esz = KIND == CacheKind::U3 ? 4 : byte_kind(KIND) ? 1 : 2;
  const int nk = (t1 - t0 + Gm::CT - 1) / Gm::CT;
  const bool ragged = ((t1 - t0) % Gm::CT) != 0;
  const int n_plain = ragged ? nk - 1 : nk;
  const int32_t* bt_row = p.block_tables + b * p.bt_sb;
  const int h_first = hg * p.heads_per_group;
  const LaneOffsets<D, HPI, KIND, G> lo = lane_offsets<D, HPI, KIND, G>(p, tr, hh, c);
  const char* kc = static_cast<const char*>(p.k_cache) + (int64_t)h_first * p.c_sh * esz;
  const char* vc = static_cast<const char*>(p.v_cache) + (int64_t)h_first * p.c_sh * esz;
  const char* kmc = static_cast<const char*>(p.k_meta) + (int64_t)h_first * p.m_sh * 4;
  const char* vmc = static_cast<const char*>(p.v_meta) + (int64_t)h_first * p.m_sh * 4;
  typedef __attribute__((address_space(3))) int LdsInt;
  LdsInt* const cnt_lds = (LdsInt*)cnt;                   // an LDS atomic (ds_add_rtn, lgkmcnt)
  // physical block ids of the request's blocks [win, win + 64), lane j <-> block win + j: one
  // vector load covers 64 blocks (1024 tokens or more), so a range reloads it rarely (a reload
  // waits for every load in flight before it); claims only grow, so the window only moves
  // forward
  const int last_blk = (t1 - 1) >> p.log2_bs;
  int win = 0, bt_lane = 0;
  bool have = false;
  // Loads of chunk k (live: k is a chunk of the range).  In the matrix-core form a chunk that is
  // not live is issued too, through resources of 0 records: every path through the loop then
  // issues the same loads, so the compiler's wait counts for the chunks in flight stay exact
  // (a load issued on one path only makes it wait for every load at the join, the ones just
  // issued included).  The row-major form skips it.
  auto issue = [&](int k, R& regs, bool live) {
    int64_t phys = 0;
    if (live) {
      const int blk = (t0 + k * Gm::CT) >> p.log2_bs;
      if (!have || blk - win >= 64) {
        win = blk;
        have = true;
        bt_lane = 0;
        if (win + lane <= last_blk) {
          const int e = bt_row[win + lane];
          bt_lane = (int)min<int64_t>(max(e, 0), p.num_blocks - 1);   // out-of-range ids clamped
        }
      }
      phys = __builtin_amdgcn_readlane(bt_lane, blk - win);
    } else if constexpr (!mq_form<D, G, HPI>()) {
      return;
    }
    const int tok0 = t0 + k * Gm::CT;
    // the chunk holding a token this workgroup appended: its rows must be in memory first (a
    // storing wave counts its own stores before it waits, so it never waits for itself)
    if (live && new_tok >= tok0 && new_tok < tok0 + Gm::CT) {
      if (app_mine) {
        count_appended(app_done);
        app_mine = false;
      }
      wait_appended(app_done, app_target);
    }
    const int64_t slot0 = tok0 & (p.block_size - 1);
    const int64_t rowb = (phys * p.c_sb + slot0 * p.c_ss) * esz;
    const int64_t metab = (phys * p.m_sb + slot0 * p.m_ss) * 4;
    load_chunk<D, HPI, KIND, G>(p, kc + rowb, vc + rowb, kmc + metab, vmc + metab, lo, c, regs, live);
  };
  auto tok_of = [&](int k) { return t0 + k * Gm::CT + tr; };
  // A ring of NB register buffers: the loads of the next NB - 1 claimed chunks are in flight
  // while one chunk is computed.  Each claim (an LDS atomic on the head wave's counter, by lane
  // 0) is issued before the chunk that precedes its use is computed, so its latency is hidden.
  // Claims only grow, so the first claim at or past n_plain (this wave's k_end) ends the
  // claiming; exactly one wave gets n_plain itself, and it takes the ragged last chunk.
  constexpr int NB = prefetch_depth<D, G, KIND, HPI>();
  int k_end = -1;
  auto claim_raw = [&]() {                        // the atomic in flight (lane 0's result)
    int v = 0;
    if (k_end < 0 && lane == 0)
      v = __hip_atomic_fetch_add(cnt_lds, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return v;
  };
  auto take = [&](int raw) {                      // the claimed chunk
    if (k_end >= 0) return k_end;
    const int k = __builtin_amdgcn_readfirstlane(raw);
    if (k >= n_plain) k_end = k;
    return k;
  };
  R r[NB];
  int kq[NB];
  int raw = claim_raw();
#pragma unroll
  for (int b = 0; b < NB - 1; ++b) {
    kq[b] = take(raw);
    raw = claim_raw();
    issue(kq[b], r[b], kq[b] < n_plain);
  }

  bool done = kq[0] >= n_plain;
  while (!done) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int nb = (b + NB - 1) % NB;           // the buffer computed last, free again
      kq[nb] = take(raw);
      raw = claim_raw();
      issue(kq[nb], r[nb], kq[nb] < n_plain);
      // keep the scheduler from hoisting this chunk's first products above the new loads: they
      // would then wait for all loads in flight before the next chunk's are even issued
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk<D, G, BF16, KIND, HPI, false>(p, S, r[b], tok_of(kq[b]), t1, c);
      if (app_mine) {                    // this wave stored appended rows: count them, one chunk on
        count_appended(app_done);
        app_mine = false;
      }
      if (kq[(b + 1) % NB] >= n_plain) {
        done = true;
        break;
      }
    }
  }
  if (app_mine) count_appended(app_done);   // a range that ended before the first computed chunk
  if (ragged && k_end == n_plain) {      // the ragged last chunk, taken by exactly one wave
    R regs;
    issue(n_plain, regs, true);
    compute_chunk<D, G, BF16, KIND, HPI, true>(p, S, regs, tok_of(n_plain), t1, c);
  }
}

// Merge the rows of the wave that hold the same head at different token offsets (TPI > 1).
template <int D, int G, CacheKind KIND, int HPI>
__device__ __forceinline__ void merge_rows(State<G>& S) {
  using Gm = Geo<D, HPI, G>;
  if constexpr (KIND == CacheKind::U3) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) PKV_ACC(S, g, e) -= S.zc[g];
  }
#pragma unroll
  for (int off = HPI * Gm::LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(S.m[g], off);
      const float lo = __shfl_xor(S.l[g], off);
      const float mn = fmaxf(S.m[g], mo);
      const float mu = (mn == neg_inf()) ? 0.f : mn;
      const float fs = fast_exp2(S.m[g] - mu), fo = fast_exp2(mo - mu);
      S.l[g] = S.l[g] * fs + lo * fo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(PKV_ACC(S, g, e), off);
        PKV_ACC(S, g, e) = PKV_ACC(S, g, e) * fs + ao * fo;
      }
      S.m[g] = mn;
    }
  }
}

// s_pref[i] = units of requests 0..i-1 (i = 0..B): a non-empty request has its granules plus
// seg_start_units units that hold no tokens, so that the static split charges the start of a
// segment (context length, q and block-table loads ahead of the first K/V) like work.
__device__ void build_prefix(const DecodeParams& p, int* s_pref, int* s_tile) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  int carry = 0;
  for (int base = 0; base < p.batch; base += blockDim.x) {
    const int i = base + threadIdx.x;
    int x = 0;
    if (i < p.batch) x = (clamp_ctx(p, i) + p.partition_size - 1) / p.partition_size;
    if (x > 0) x += p.seg_start_units;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_tile[w] = x;
    __syncthreads();
    int before = carry, total = carry;
    for (int j = 0; j < nwv; ++j) {
      if (j < w) before += s_tile[j];
      total += s_tile[j];
    }
    if (i < p.batch) s_pref[i + 1] = before + x;
    carry = total;
    __syncthreads();
  }
  if (threadIdx.x == 0) s_pref[0] = 0;
  __syncthreads();
}

template <bool BF16>
__device__ __forceinline__ void store_out_row(const DecodeParams& p, int b, int h, int c,
                                              const float (&a)[8], float inv_l) {
  uint4 o;
  o.x = pack2<BF16>(a[0] * inv_l, a[1] * inv_l);
  o.y = pack2<BF16>(a[2] * inv_l, a[3] * inv_l);
  o.z = pack2<BF16>(a[4] * inv_l, a[5] * inv_l);
  o.w = pack2<BF16>(a[6] * inv_l, a[7] * inv_l);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + b * p.o_sb + (int64_t)h * p.o_sh + c * 8) = o;
}

// The fused append of a decode step ("Write Triton Kv Cache Append Kernel", Required reasoning
// process steps 4-9, with the slot of request b's new token taken from its block table as step 9
// builds it: block_tables[b, pos / block_size] * block_size + pos % block_size, pos =
// context_lens[b] - 1): the new K and V rows of the group's heads, converted to the cache's format
// as kv_append converts them (append_rows.cuh).  A block id outside the pool skips the write, as
// kv_append skips a slot outside the pool.  Called by the one workgroup that reads that token.
// The rows are loaded together with the block id (one load latency).  Each wave that holds rows
// later waits for its own stores to complete and counts itself done in an LDS counter (in
// run_range, after its first computed chunk, by when the stores have long completed); the wave
// that loads the chunk holding the new token waits for that count first (wait_appended), so no
// other wave waits and no barrier is needed.  Returns the number of waves that store.
template <int D, bool BF16, CacheKind KIND>
__device__ __forceinline__ int append_new_rows(const DecodeParams& p, int b, int hg, int ctx) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;                          // rows per wave
  const int pos = ctx - 1;
  const int e = p.block_tables[(int64_t)b * p.bt_sb + (pos >> p.log2_bs)];
  const int64_t off = pos & (p.block_size - 1);
  const int c = threadIdx.x % LPR;
  const int nwaves = blockDim.x >> 6;
  const int storing = min(nwaves, (p.heads_per_group + RPW - 1) / RPW);
  for (int r = threadIdx.x / LPR; r < p.heads_per_group; r += blockDim.x / LPR) {
    const int h = hg * p.heads_per_group + r;
    const uint4 kx = load_stream_u4(static_cast<const uint16_t*>(p.k_new) + b * p.kn_sb + (int64_t)h * p.kn_sh + c * 8);
    const uint4 vx = load_stream_u4(static_cast<const uint16_t*>(p.v_new) + b * p.vn_sb + (int64_t)h * p.vn_sh + c * 8);
    if (e >= 0 && e < p.num_blocks) {                   // the same value in every lane
      const int64_t crow = (int64_t)e * p.c_sb + off * p.c_ss + (int64_t)h * p.c_sh;
      const int64_t mrow = (int64_t)e * p.m_sb + off * p.m_ss + (int64_t)h * p.m_sh;
      store_kv_row<LPR, BF16, KIND>(kx, vx, const_cast<void*>(p.k_cache), const_cast<void*>(p.v_cache),
                                    const_cast<void*>(p.k_meta), const_cast<void*>(p.v_meta), crow, mrow, c,
                                    false);
    }
  }
  return storing;
}

template <int D, int G, bool BF16, CacheKind KIND, int HPI>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_kernel(DecodeParams p) {
  using Gm = Geo<D, HPI, G>;
  extern __shared__ int s_pref[];              // batch + 1 entries
  __shared__ int s_tile[kMaxWaves];
  // chunk counters of the head waves' token streams, one set per segment parity: the set of
  // segment i + 1 is cleared during segment i, after the barriers that end segment i - 1
  __shared__ int s_cnt[2][kMaxWaves];
  // waves whose rows of a fused append have reached memory (counts up over the segments)
  __shared__ int s_app_done;
  if (threadIdx.x < 2 * kMaxWaves) s_cnt[threadIdx.x / kMaxWaves][threadIdx.x % kMaxWaves] = 0;
  if (threadIdx.x == 0) s_app_done = 0;
  build_prefix(p, s_pref, s_tile);             // (ends with a barrier)

  const int lane = threadIdx.x & 63;
  const int hw_count = p.heads_per_group / HPI;  // waves per token stream
  const int wv = (threadIdx.x >> 6) % hw_count;  // wave inside the token stream
  const int stream = (threadIdx.x >> 6) / hw_count;
  const int r = lane / Gm::LPR;
  const int c = lane % Gm::LPR;
  const int hr = r % HPI;                       // head of the row inside the instruction
  const int tr = r / HPI;                       // token offset of the row
  // token streams 1.. hand their per-segment state to stream 0 through LDS:
  // [stream - 1][head in group][query head][D accumulators, m, l]
  float* s_x = reinterpret_cast<float*>(s_pref + ((p.batch + 1 + 3) & ~3));
  const int64_t NHG = p.num_head_groups;
  const int64_t total = NHG * s_pref[p.batch];            // units of all segments
  const int64_t wg = blockIdx.x;
  int64_t x = range_start(p, total, wg);
  const int64_t x_end = range_start(p, total, wg + 1);
  if (x == x_end) {            // empty range (fewer units than workgroups): an empty state in slot 0
    const int n_st = p.heads_per_group * G;
    for (int i = threadIdx.x; i < n_st * D; i += blockDim.x) p.ws_acc[(wg * 2 * n_st) * D + i] = 0.f;
    for (int i = threadIdx.x; i < n_st; i += blockDim.x)
      *reinterpret_cast<float2*>(p.ws_ml + (wg * 2 * n_st + i) * 2) = make_float2(neg_inf(), 0.f);
    return;
  }
  bool first = true;
  int seg_i = 0;
  int app_target = 0;                           // s_app_done once this workgroup's appends are in
  while (x < x_end) {
    // segment (request b, head group hg) holding unit x: the last b with NHG*s_pref[b] <= x
    int lo = 0, hi = p.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (NHG * s_pref[mid] <= x) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int n = s_pref[b + 1] - s_pref[b];
    const int64_t off = x - NHG * s_pref[b];
    const int hg = (int)(off / n);
    const int g0 = (int)(off - (int64_t)hg * n);
    const int g1 = (int)min<int64_t>(n, g0 + (x_end - x));
    const int ctx = clamp_ctx(p, b);
    if (threadIdx.x == 0) {                    // where the merge kernel finds this segment's pieces
      const int64_t sidx = (int64_t)b * NHG + hg;
      if (g0 == 0) p.ws_seg[2 * sidx] = (int)(wg * 2 + (first ? 0 : 1));
      if (g1 == n) p.ws_seg[2 * sidx + 1] = (int)wg;
    }
    const int t0 = max(g0 - p.seg_start_units, 0) * p.partition_size;   // start units: no tokens
    const int t1 = min(ctx, max(g1 - p.seg_start_units, 0) * p.partition_size);
    const int hh = wv * HPI + hr;                          // head inside the group
    const int h = hg * p.heads_per_group + hh;             // kv head of this lane's row

    State<G> S;
    constexpr bool MQ = mq_form<D, G, HPI>();
    const uint16_t* q_row = static_cast<const uint16_t*>(p.q) + b * p.q_sb + (int64_t)h * G * p.q_sh;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      S.qsum[g] = 0.f;
      S.m[g] = neg_inf();
      S.l[g] = 0.f;
      S.zc[g] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) PKV_ACC(S, g, e) = 0.f;
      if constexpr (MQ) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(q_row + (int64_t)g * p.q_sh + c * 8);
      if constexpr (KIND == CacheKind::U3) {
        // pairs (q[e], q[e + 4]) of the lane's 8 elements, the order the 3-bit codes unpack in
        S.qv[g][0] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
        S.qv[g][1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
        S.qv[g][2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
        S.qv[g][3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
      } else {
        S.qv[g][0] = v.x; S.qv[g][1] = v.y; S.qv[g][2] = v.z; S.qv[g][3] = v.w;
      }
      if constexpr (KIND == CacheKind::U3) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) s += h_lo<BF16>(S.qv[g][e]) + h_hi<BF16>(S.qv[g][e]);
        S.qsum[g] = group_sum<Gm::LPR>(s);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      S.mo[h] = neg_inf();
      S.lo[h] = 0.f;
      S.zco[h] = 0.f;
      // the query sums of the lane's own heads (q mod G, or q and q + 4 with 8 heads)
      const int own = (G == 8) ? (lane & 3) + 4 * h : (lane & 3 & (G - 1));
      S.qso[h] = S.qsum[0];
#pragma unroll
      for (int g = 1; g < G; ++g)
        if (own == g) S.qso[h] = S.qsum[g];
    }
    if constexpr (MQ) {
      // B operands of the score products: the lane's column head (lane mod 4, with 8 heads also
      // + 4) at the head-dim slice j of each load instruction i; 3-bit: pairs (q[e], q[e + 4]),
      // the order its codes unpack in, and the head's query sum for the zero point
#pragma unroll
      for (int hs = 0; hs < own_heads<G>(); ++hs) {
        const int g = (G == 8) ? (lane & 3) + 4 * hs : (lane & 3 & (G - 1));
        float qs = 0.f;
#pragma unroll
        for (int i = 0; i < Gm::NI; ++i) {
          const int j = mq_slice<Gm::LPR, KIND>(i, c >> 2);
          const uint4 v = *reinterpret_cast<const uint4*>(q_row + (int64_t)g * p.q_sh + j * 8);
          if constexpr (KIND == CacheKind::U3) {
            S.qm[hs][i][0] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
            S.qm[hs][i][1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
            S.qm[hs][i][2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
            S.qm[hs][i][3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
#pragma unroll
            for (int e = 0; e < 4; ++e) qs += h_lo<BF16>(S.qm[hs][i][e]) + h_hi<BF16>(S.qm[hs][i][e]);
          } else {
            S.qm[hs][i][0] = v.x; S.qm[hs][i][1] = v.y; S.qm[hs][i][2] = v.z; S.qm[hs][i][3] = v.w;
          }
        }
        // fp16 scores are taken with the 3-bit codes as code * 2^-24 (exactly): the query sum
        // is kept in the same units
        if constexpr (KIND == CacheKind::U3) S.qso[hs] = row_quads_sum<Gm::LPR>(qs) * (BF16 ? 1.f : 0x1p-24f);
      }
    }
    if (seg_i > 0 && threadIdx.x < kMaxWaves) s_cnt[(seg_i + 1) & 1][threadIdx.x] = 0;
    int* cnt = &s_cnt[seg_i & 1][wv];
    int new_tok = -1;
    bool app_mine = false;                      // this wave stored rows of this segment's append
    if (p.k_new != nullptr && g1 == n) {
      // fused append: this workgroup holds the segment's last granule, so it alone reads the new
      // token, at position ctx - 1; the wave that loads it waits for the rows (append_new_rows)
      const int storing = append_new_rows<D, BF16, KIND>(p, b, hg, ctx);
      app_target += storing;
      app_mine = (int)(threadIdx.x >> 6) < storing;
      new_tok = ctx - 1;
    }
    run_range<D, G, BF16, KIND, HPI>(p, S, b, hg, t0, t1, lane, tr, hh, c, cnt, new_tok, &s_app_done,
                                     app_target, app_mine);
    if constexpr (own_head_form<D, G>()) {      // every head's running sums into every lane
      quad_gather<G>(S.lo, S.l);
      if constexpr (KIND == CacheKind::U3) quad_gather<G>(S.zco, S.zc);
    }
    merge_rows<D, G, KIND, HPI>(S);
    if (p.token_streams > 1) {
      if (stream > 0 && tr == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float* xs = s_x + (((int64_t)(stream - 1) * p.heads_per_group + hh) * G + g) * (D + 2);
#pragma unroll
          for (int e = 0; e < 8; ++e) xs[c * 8 + e] = PKV_ACC(S, g, e);
          if (c == 0) {
            xs[D] = S.m[g];
            xs[D + 1] = S.l[g];
          }
        }
      }
      __syncthreads();
      if (stream == 0) {
        for (int q = 1; q < p.token_streams; ++q) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float* xs = s_x + (((int64_t)(q - 1) * p.heads_per_group + hh) * G + g) * (D + 2);
            const float mo = xs[D], lo2 = xs[D + 1];
            const float mn = fmaxf(S.m[g], mo);
            const float mu = (mn == neg_inf()) ? 0.f : mn;
            const float fs = fast_exp2(S.m[g] - mu), fo = fast_exp2(mo - mu);
            S.l[g] = S.l[g] * fs + lo2 * fo;
#pragma unroll
            for (int e = 0; e < 8; ++e) PKV_ACC(S, g, e) = PKV_ACC(S, g, e) * fs + xs[c * 8 + e] * fo;
            S.m[g] = mn;
          }
        }
      }
      __syncthreads();                          // the buffer is reused by the next segment
    }
    if (stream == 0 && tr == 0) {
      if (g0 == 0 && g1 == n) {                   // whole segment: final output
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) a8[e] = PKV_ACC(S, g, e);
          store_out_row<BF16>(p, b, h * G + g, c, a8, 1.f / S.l[g]);
        }
      } else {                                    // part of a split segment
        const int64_t slot = (wg * 2 + (first ? 0 : 1)) * p.heads_per_group + hh;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float* dst = p.ws_acc + (slot * G + g) * D + c * 8;
          *reinterpret_cast<float4*>(dst) = make_float4(PKV_ACC(S, g, 0), PKV_ACC(S, g, 1), PKV_ACC(S, g, 2), PKV_ACC(S, g, 3));
          *reinterpret_cast<float4*>(dst + 4) = make_float4(PKV_ACC(S, g, 4), PKV_ACC(S, g, 5), PKV_ACC(S, g, 6), PKV_ACC(S, g, 7));
          if (c == 0) *reinterpret_cast<float2*>(p.ws_ml + (slot * G + g) * 2) = make_float2(S.m[g], S.l[g]);
        }
      }
    }
    x += g1 - g0;
    first = false;
    ++seg_i;
  }
}

// ---------------------------------------------------------------------------------------
// Instance lookup.  The instances are compiled in ten translation units (decode_{same, fp8,
// e5m2, i8, u3}_d{128, 64}), each exporting the pointer lookup of its head dim and cache kind,
// so that the build can compile them in parallel.
// ---------------------------------------------------------------------------------------
template <int D, int G, bool BF16, CacheKind KIND, int HPI>
const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&decode_kernel<D, G, BF16, KIND, HPI>);
}

template <int D, int G, bool BF16, CacheKind KIND>
const void* kernel_by_hpi(int hpi) {
  switch (hpi) {
    case 1: return kernel_ptr<D, G, BF16, KIND, 1>();
    case 2: return kernel_ptr<D, G, BF16, KIND, 2>();
    case 4: return kernel_ptr<D, G, BF16, KIND, 4>();
    case 8: if constexpr (D == 64) return kernel_ptr<D, G, BF16, KIND, 8>(); else return nullptr;
  }
  return nullptr;
}

template <int D, bool BF16, CacheKind KIND>
const void* kernel_by_g(int group, int hpi) {
  switch (group) {
    case 1: return kernel_by_hpi<D, 1, BF16, KIND>(hpi);
    case 2: return kernel_by_hpi<D, 2, BF16, KIND>(hpi);
    case 4: return kernel_by_hpi<D, 4, BF16, KIND>(hpi);
    case 8: return kernel_by_hpi<D, 8, BF16, KIND>(hpi);
  }
  return nullptr;
}

template <int D, CacheKind KIND>
const void* kernel_by_dtype(int group, bool bf16, int hpi) {
  return bf16 ? kernel_by_g<D, true, KIND>(group, hpi) : kernel_by_g<D, false, KIND>(group, hpi);
}

// host pointer of decode_kernel<D, group, bf16, KIND, hpi>, or nullptr if not built
const void* decode_kernel_ptr_same_d128(int group, bool bf16, int hpi);
const void* decode_kernel_ptr_same_d64(int group, bool bf16, int hpi);
const void* decode_kernel_ptr_fp8_d128(int group, bool bf16, int hpi);
const void* decode_kernel_ptr_fp8_d64(int group, bool bf16, int hpi);
const void* decode_kernel_ptr_u3_d128(int group, bool bf16, int hpi);
const void* decode_kernel_ptr_u3_d64(int group, bool bf16, int hpi);
const void* decode_kernel_ptr_e5m2_d128(int group, bool bf16, int hpi);
const void* decode_kernel_ptr_e5m2_d64(int group, bool bf16, int hpi);
const void* decode_kernel_ptr_i8_d128(int group, bool bf16, int hpi);
const void* decode_kernel_ptr_i8_d64(int group, bool bf16, int hpi);

}  // namespace pkv

// Internal launchers behind the C ABI (validated arguments only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum class CacheKind : int { Same = 0, Fp8 = 1, U3 = 2, E5m2 = 3, I8 = 4 };
constexpr int kNumCacheKinds = 5;
// caches of one byte code per element with one fp32 scale per row: fp8 e4m3fn, fp8 e5m2, int8
constexpr bool byte_kind(CacheKind k) {
  return k == CacheKind::Fp8 || k == CacheKind::E5m2 || k == CacheKind::I8;
}

struct AppendParams {
  const void* k_new;
  const void* v_new;
  int64_t k_st, k_sh, v_st, v_sh;     // elements
  const int64_t* slots;
  int64_t num_tokens;
  void* k_cache;
  void* v_cache;
  int64_t c_sb, c_ss, c_sh;           // elements (bytes for byte codes, words for u3)
  void* k_meta;
  void* v_meta;
  int64_t m_sb, m_ss, m_sh;           // meta entry of row (blk, slot, head): blk*m_sb + slot*m_ss + head*m_sh
  int given_scale;                    // byte codes: 1 = read the caller's scales, 0 = compute and write
  int64_t capacity;                   // num_blocks * block_size
  int log2_bs;
  int num_kv_heads;
};

struct DecodeParams {
  void* out;
  const void* q;
  int64_t q_sb, q_sh, o_sb, o_sh;     // elements
  const void* k_cache;
  const void* v_cache;
  int64_t c_sb, c_ss, c_sh;           // elements (words for u3)
  const void* k_meta;                 // u3: fp16 (s, z) per row; byte codes: fp32 scales
  const void* v_meta;
  int64_t m_sb, m_ss, m_sh;           // meta entry of row (blk, slot, head): blk*m_sb + slot*m_ss + head*m_sh
  const int32_t* block_tables;
  int64_t bt_sb;
  const int32_t* context_lens;
  int num_q_heads, num_kv_heads;
  int batch;
  int block_size, log2_bs;
  int64_t num_blocks;                 // block-table entries are clamped into [0, num_blocks)
  int max_context_len;                // context lengths are clamped into [0, max_context_len]
  int partition_size;                 // split granule in tokens, multiple of 16
  int seg_start_units;                // units without tokens ahead of each non-empty segment
  int64_t num_wgs;                    // workgroups in the decode grid
  int64_t split_tier;                 // workgroups of the first dispatch tier (one per CU)
  int64_t split_w[4];                 // units share of workgroup w: [tier * 2 + (w & 1)]
  int heads_per_group;                // kv heads one workgroup covers
  int num_head_groups;                // num_kv_heads / heads_per_group
  int token_streams;                  // waves sets of a workgroup splitting its chunks
  float scale_log2;                   // sm_scale * log2(e)
  // 3-bit PV operands: the mask of bits 7..9 of each 16-bit half and the fp16 8.0 pair.  Passed
  // in rather than written as literals, so that the compiler can fuse the mask and the bias into
  // one three-operand instruction (whose encoding here takes no literal)
  uint32_t u3_code_mask, u3_code_bias;
  float* ws_acc;                      // [num_wgs, 2, heads_per_group, G, D] partial accumulators
  float* ws_ml;                       // [num_wgs, 2, heads_per_group, G, 2] partial (m, l)
  int* ws_seg;                        // [batch, head groups, 2] first partial slot, last owner
  // fused append of a decode step (paged_decode_append): request b's new K and V rows,
  // [batch, num_kv_heads, head_dim] of the query dtype, are written at position
  // context_lens[b] - 1 before the decode reads it; nullptr: no append
  const void* k_new;
  const void* v_new;
  int64_t kn_sb, kn_sh, vn_sb, vn_sh; // elements
};

struct SlotParams {
  const int32_t* token_request;       // nullptr: token t belongs to request t
  const int32_t* token_position;
  int64_t num_tokens;
  const int32_t* block_tables;        // nullptr: contiguous cache, slot = request * 2^log2_bs + position
  int64_t bt_sb;
  int batch;
  int log2_bs;
  int64_t* slot_mapping;
};

// Launch geometry of paged_decode.
struct DecodePlan {
  int hpi;                            // kv heads per wave instruction
  int waves_per_wg;
  int heads_per_group;                // hpi * (waves_per_wg / token_streams)
  int num_head_groups;
  int token_streams;                  // waves per head wave sharing out its chunks
  int64_t num_wgs;                    // as many as stay resident, at most one per unit
  int64_t split_tier;                 // first dispatch tier: min(num_wgs, compute units)
  int chunk_tokens;                   // tokens per chunk of a token stream
  size_t lds_bytes;                   // dynamic LDS of the decode kernel
};

hipError_t launch_slots(const SlotParams& p, hipStream_t s);
hipError_t launch_pack3(const uint8_t* values, uint8_t* packed, int64_t n_values, hipStream_t s);
hipError_t launch_unpack3(const uint8_t* packed, uint8_t* values, int64_t n_values, hipStream_t s);

// bf16: true for bfloat16 inputs, false for fp16.
hipError_t launch_append(const AppendParams& p, CacheKind kind, bool bf16, int head_dim,
                         hipStream_t s);

hipError_t launch_decode(const DecodeParams& p, const DecodePlan& plan, CacheKind kind, bool bf16,
                         int head_dim, int group, hipStream_t s);

// Split granule used when the caller passes 0.
int auto_partition_size(int max_context_len, int batch, int num_q_heads);

// Launch geometry on the current device; kind is a CacheKind value.  bf16 / kind = -1 plans
// for the largest grid any dtype or cache kind would use (for sizing a workspace).
DecodePlan plan_decode(int batch, int num_q_heads, int num_kv_heads, int head_dim, int max_context_len,
                       int partition_size, int bf16, int kind);

}  // namespace pkv

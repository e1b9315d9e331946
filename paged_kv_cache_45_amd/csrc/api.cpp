// C ABI entry points: host-side validation, then dispatch to the HIP launchers.
// Every check runs before anything is enqueued; a failing call writes nothing.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstddef>
#include <mutex>

#include "../../include/pagedkv.h"
#include "launch.h"

using pkv::CacheKind;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

// head_dim / block_size: malformed (<= 0 or not a power of two) is EINVAL, a well-formed
// value outside the compiled set is EUNSUPPORTED.
int check_head_dim(int d) {
  if (d <= 0) return PKV_EINVAL;
  return (d == 64 || d == 128) ? PKV_OK : PKV_EUNSUPPORTED;
}
int check_block_size(int bs) {
  if (bs <= 0 || log2_exact(bs) < 0) return PKV_EINVAL;
  return (bs == 16 || bs == 32 || bs == 64) ? PKV_OK : PKV_EUNSUPPORTED;
}
// The append and the slot builder take any power-of-two block from 16 to 2^24 tokens: the
// contiguous cache is the pool whose block is one request's whole sequence.
constexpr int kMaxAppendBlock = 1 << 24;
int check_append_block_size(int bs) {
  if (bs <= 0 || log2_exact(bs) < 0) return PKV_EINVAL;
  return (bs >= 16 && bs <= kMaxAppendBlock) ? PKV_OK : PKV_EUNSUPPORTED;
}
bool is16(pkv_dtype t) { return t == PKV_F16 || t == PKV_BF16; }
bool known(pkv_dtype t) {
  return t == PKV_F16 || t == PKV_BF16 || t == PKV_FP8_E4M3FN || t == PKV_U3 || t == PKV_FP8_E5M2 ||
         t == PKV_INT8;
}
// one byte code per element and one fp32 scale per row
bool is_byte_code(pkv_dtype t) { return t == PKV_FP8_E4M3FN || t == PKV_FP8_E5M2 || t == PKV_INT8; }
CacheKind byte_cache_kind(pkv_dtype t) {
  return t == PKV_FP8_E5M2 ? CacheKind::E5m2 : t == PKV_INT8 ? CacheKind::I8 : CacheKind::Fp8;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int resolve_partition(int partition_size, int max_context_len, int batch, int num_q_heads) {
  return partition_size == 0 ? pkv::auto_partition_size(max_context_len, batch, num_q_heads)
                             : partition_size;
}

constexpr int kMaxPartition = 1 << 20;
constexpr int kMaxBatch = 8192;       // the decode kernel keeps batch + 1 prefix sums in LDS
// Static split weights (units share of a workgroup, in 1/64), by dispatch tier (the first
// workgroup on each CU streams ahead of the CU's later ones) and by the parity of its XCD
// (workgroup w runs on XCD w mod 8; per-workgroup traces of the Llama-8B step showed the
// odd-numbered XCDs ending 5 % later on average, on three machines).  Measured, three
// interleaved runs each:
//  * static split, bf16/fp16 cache (HBM-bound): first tier 96 (24/16), odd 61 against 88 / 64:
//    Llama-8B step 0.602 -> 0.607 of HBM peak;
//  * static split, 3-bit cache (VALU-bound, so the XCDs' memory paths do not matter): first
//    tier 96 helps (+0.4 %), the odd-XCD weight costs 1 %;
//  * long-context decode (64-token blocks, 32k-128k contexts): 88 / 64 and 96 / 92 / 64 / 61
//    equal within noise.
struct SplitWeights { int64_t first_even, first_odd, rest_even, rest_odd; };
constexpr SplitWeights kSplitStatic{96, 92, 64, 61};
constexpr SplitWeights kSplitStaticU3{96, 96, 64, 64};
// a workgroup that starts a segment inside its range first waits for the segment's context
// length, q and block table: charged to the static split as this many tokens of work
// (measured with one 8-wave workgroup per CU: 16 -> 48 gains 1 % on the Llama-8B step, 2 % on
// the 3-bit decode; 32 and 48 are equal on the former).  A coded-cache token costs about half a
// 16-bit one or less, so the same wait is worth more of them: 96 measured best for fp8, e5m2
// and int8 at the Llama-8B shape (+0.6-0.9 %, +1.0 %, +1.8-2.5 % against 48; 24, 144 and 192
// slower) and for the 3-bit decode with its 16-bit PV products (+0.9 %).
constexpr int kSegmentStartTokens = 48;
constexpr int kSegmentStartTokensCoded = 96;

struct DecodeLayout {
  pkv::DecodePlan plan;
  size_t acc_off, ml_off, seg_off, bytes;
};

// Workspace layout of paged_decode: the partial accumulators, the partial (m, l), and per
// segment (request, kv-head group) the slot of its first partial and the owner of its last unit.
// Every call writes each part before it reads it, so the workspace needs no particular contents
// and one workspace serves calls of every shape it is large enough for.
DecodeLayout decode_layout(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                           int max_context_len, int ps, int bf16, int kind) {
  DecodeLayout L{};
  const int64_t group = num_q_heads / num_kv_heads;
  L.plan = pkv::plan_decode(batch, num_q_heads, num_kv_heads, head_dim, max_context_len, ps, bf16, kind);
  const size_t slots = (size_t)L.plan.num_wgs * 2 * L.plan.heads_per_group * group;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L.acc_off = 0;
  L.ml_off = L.acc_off + up(slots * head_dim * sizeof(float));
  L.seg_off = L.ml_off + up(slots * 2 * sizeof(float));
  L.bytes = L.seg_off + up((size_t)batch * L.plan.num_head_groups * 2 * sizeof(int));
  return L;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported configuration";
    case PKV_EWORKSPACE: return "workspace missing or too small";
    case PKV_EHIP: return "HIP launch failed";
    case PKV_ESCRATCH: return "the call needs more decode scratch than the static buffer holds";
    default: return "unknown status";
  }
}

int build_slot_mapping(const int32_t* token_request, const int32_t* token_position, int64_t num_tokens,
                       const int32_t* block_tables, int64_t bt_stride_b, int batch, int block_size,
                       int64_t* slot_mapping, hipStream_t stream) {
  if (num_tokens < 0 || batch < 0) return PKV_EINVAL;
  if (num_tokens >= (int64_t(1) << 31)) return PKV_EUNSUPPORTED;
  const int st = check_append_block_size(block_size);
  if (st != PKV_OK) return st;
  if (num_tokens == 0) return PKV_OK;
  if (!token_position || !slot_mapping || !aligned(token_position, 4) || !aligned(slot_mapping, 8))
    return PKV_EINVAL;
  if (token_request && !aligned(token_request, 4)) return PKV_EINVAL;
  if (block_tables && (!aligned(block_tables, 4) || bt_stride_b <= 0)) return PKV_EINVAL;
  pkv::SlotParams p{};
  p.token_request = token_request;
  p.token_position = token_position;
  p.num_tokens = num_tokens;
  p.block_tables = block_tables;
  p.bt_sb = bt_stride_b;
  p.batch = batch;
  p.log2_bs = log2_exact(block_size);
  p.slot_mapping = slot_mapping;
  return pkv::launch_slots(p, stream) == hipSuccess ? PKV_OK : PKV_EHIP;
}

int pack3(const uint8_t* values, uint8_t* packed, int64_t n_values, hipStream_t stream) {
  if (n_values < 0 || n_values % 8) return PKV_EINVAL;
  if (n_values == 0) return PKV_OK;
  if (!values || !packed) return PKV_EINVAL;
  return pkv::launch_pack3(values, packed, n_values, stream) == hipSuccess ? PKV_OK : PKV_EHIP;
}

int unpack3(const uint8_t* packed, uint8_t* values, int64_t n_values, hipStream_t stream) {
  if (n_values < 0 || n_values % 8) return PKV_EINVAL;
  if (n_values == 0) return PKV_OK;
  if (!values || !packed) return PKV_EINVAL;
  return pkv::launch_unpack3(packed, values, n_values, stream) == hipSuccess ? PKV_OK : PKV_EHIP;
}

// kv_append and kv_append_scaled.  The meta entry (scale, or u3 scale/zero) of row (blk, slot,
// head) is m_sb*blk + m_ss*slot + m_sh*head; given: the caller's scales are read, not written.
static int append_impl(const void* k_new, const void* v_new, pkv_dtype in_dtype,
                       int64_t k_stride_tok, int64_t k_stride_head,
                       int64_t v_stride_tok, int64_t v_stride_head,
                       const int64_t* slot_mapping, int64_t num_tokens,
                       void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                       int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                       void* k_meta, void* v_meta,
                       int64_t num_blocks, int block_size, int num_kv_heads, int head_dim,
                       hipStream_t stream, int64_t m_sb, int64_t m_ss, int64_t m_sh, bool given) {
  if (!known(in_dtype) || !known(cache_dtype)) return PKV_EINVAL;
  if (given && !is_byte_code(cache_dtype)) return PKV_EINVAL;
  if (m_sb < 0 || m_ss < 0 || m_sh < 0) return PKV_EINVAL;
  if (!is16(in_dtype)) return PKV_EUNSUPPORTED;
  // a 16-bit cache must have the input's dtype (no implicit fp16 <-> bf16 conversion)
  if (is16(cache_dtype) && cache_dtype != in_dtype) return PKV_EINVAL;
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PKV_EINVAL;
  // rows (token, kv head) are indexed in 32 bits (2^31 rows of >= 128 bytes exceed any GPU)
  if (num_tokens >= (int64_t(1) << 31) / num_kv_heads) return PKV_EUNSUPPORTED;
  int st = check_head_dim(head_dim);
  if (st != PKV_OK) return st;
  st = check_append_block_size(block_size);
  if (st != PKV_OK) return st;
  if (num_tokens == 0) return PKV_OK;   // nothing to read or write (source pointers may be NULL)
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_EINVAL;
  if (k_stride_tok < 0 || k_stride_head < 0 || v_stride_tok < 0 || v_stride_head < 0 ||
      c_stride_block < 0 || c_stride_slot < 0 || c_stride_head < 0)
    return PKV_EINVAL;
  // 16-byte source rows (8 elements per lane)
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || k_stride_tok % 8 || k_stride_head % 8 ||
      v_stride_tok % 8 || v_stride_head % 8)
    return PKV_EINVAL;
  if (!aligned(slot_mapping, 8)) return PKV_EINVAL;
  CacheKind kind = CacheKind::Same;
  if (is_byte_code(cache_dtype)) {
    kind = byte_cache_kind(cache_dtype);
    if (!aligned(k_cache, 8) || !aligned(v_cache, 8) || c_stride_block % 8 || c_stride_slot % 8 ||
        c_stride_head % 8)
      return PKV_EINVAL;
    if (!k_meta || !v_meta || !aligned(k_meta, 4) || !aligned(v_meta, 4)) return PKV_EINVAL;
  } else if (cache_dtype == PKV_U3) {
    kind = CacheKind::U3;
    if (!aligned(k_cache, 4) || !aligned(v_cache, 4)) return PKV_EINVAL;
    if (!k_meta || !v_meta || !aligned(k_meta, 4) || !aligned(v_meta, 4)) return PKV_EINVAL;
  } else {
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || c_stride_block % 8 ||
        c_stride_slot % 8 || c_stride_head % 8)
      return PKV_EINVAL;
  }
  pkv::AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_st = k_stride_tok;
  p.k_sh = k_stride_head;
  p.v_st = v_stride_tok;
  p.v_sh = v_stride_head;
  p.slots = slot_mapping;
  p.num_tokens = num_tokens;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.c_sb = c_stride_block;
  p.c_ss = c_stride_slot;
  p.c_sh = c_stride_head;
  p.k_meta = k_meta;
  p.v_meta = v_meta;
  p.m_sb = m_sb;
  p.m_ss = m_ss;
  p.m_sh = m_sh;
  p.given_scale = given ? 1 : 0;
  p.capacity = num_blocks * block_size;
  p.log2_bs = log2_exact(block_size);
  p.num_kv_heads = num_kv_heads;
  const hipError_t e = pkv::launch_append(p, kind, in_dtype == PKV_BF16, head_dim, stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

int kv_append(const void* k_new, const void* v_new, pkv_dtype in_dtype,
              int64_t k_stride_tok, int64_t k_stride_head,
              int64_t v_stride_tok, int64_t v_stride_head,
              const int64_t* slot_mapping, int64_t num_tokens,
              void* k_cache, void* v_cache, pkv_dtype cache_dtype,
              int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
              void* k_meta, void* v_meta,
              int64_t num_blocks, int block_size, int num_kv_heads, int head_dim,
              hipStream_t stream) {
  // one meta entry per row, [num_blocks, block_size, num_kv_heads]
  return append_impl(k_new, v_new, in_dtype, k_stride_tok, k_stride_head, v_stride_tok, v_stride_head,
                     slot_mapping, num_tokens, k_cache, v_cache, cache_dtype, c_stride_block,
                     c_stride_slot, c_stride_head, k_meta, v_meta, num_blocks, block_size,
                     num_kv_heads, head_dim, stream, (int64_t)block_size * num_kv_heads, num_kv_heads,
                     1, false);
}

int kv_append_scaled(const void* k_new, const void* v_new, pkv_dtype in_dtype,
                     int64_t k_stride_tok, int64_t k_stride_head,
                     int64_t v_stride_tok, int64_t v_stride_head,
                     const int64_t* slot_mapping, int64_t num_tokens,
                     void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                     int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                     const float* k_scale, const float* v_scale,
                     int64_t s_stride_block, int64_t s_stride_slot, int64_t s_stride_head,
                     int64_t num_blocks, int block_size, int num_kv_heads, int head_dim,
                     hipStream_t stream) {
  return append_impl(k_new, v_new, in_dtype, k_stride_tok, k_stride_head, v_stride_tok, v_stride_head,
                     slot_mapping, num_tokens, k_cache, v_cache, cache_dtype, c_stride_block,
                     c_stride_slot, c_stride_head, const_cast<float*>(k_scale),
                     const_cast<float*>(v_scale), num_blocks, block_size, num_kv_heads, head_dim,
                     stream, s_stride_block, s_stride_slot, s_stride_head, true);
}

size_t paged_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                   int max_context_len, int partition_size) {
  if (batch < 0 || batch > kMaxBatch || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || max_context_len < 0 || check_head_dim(head_dim) != PKV_OK)
    return (size_t)-1;
  if (partition_size < 0 || partition_size % 16 || partition_size > kMaxPartition)
    return (size_t)-1;
  const int ps = resolve_partition(partition_size, max_context_len, batch, num_q_heads);
  if (batch == 0) return 0;
  return decode_layout(batch, num_q_heads, num_kv_heads, head_dim, max_context_len, ps, -1, -1).bytes;
}

// The new K and V rows of a fused decode step (paged_decode_append): [batch, num_kv_heads,
// head_dim] of the query dtype, element strides.
struct NewRows {
  const void* k;
  const void* v;
  int64_t k_sb, k_sh, v_sb, v_sh;
};

// paged_decode, paged_decode_scaled and paged_decode_append (new rows given); meta entry of row
// (blk, slot, head) as for append_impl.
static int decode_impl(void* out, const void* q, pkv_dtype q_dtype,
                       int64_t q_stride_b, int64_t q_stride_h, int64_t o_stride_b, int64_t o_stride_h,
                       const void* k_cache, const void* v_cache, pkv_dtype cache_dtype,
                       int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                       const void* k_meta, const void* v_meta,
                       const int32_t* block_tables, int64_t bt_stride_b, const int32_t* context_lens,
                       int batch, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                       int64_t num_blocks, int max_context_len, float sm_scale, int partition_size,
                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                       int64_t m_sb, int64_t m_ss, int64_t m_sh, const NewRows* nr = nullptr) {
  if (!known(q_dtype) || !known(cache_dtype)) return PKV_EINVAL;
  if (nr) {                            // the fused append's new rows: 16-byte rows of the query dtype
    if (!nr->k || !nr->v || !aligned(nr->k, 16) || !aligned(nr->v, 16)) return PKV_EINVAL;
    if (nr->k_sb < 0 || nr->k_sh < 0 || nr->v_sb < 0 || nr->v_sh < 0 || nr->k_sb % 8 || nr->k_sh % 8 ||
        nr->v_sb % 8 || nr->v_sh % 8)
      return PKV_EINVAL;
  }
  if (m_sb < 0 || m_ss < 0 || m_sh < 0) return PKV_EINVAL;
  if (!is16(q_dtype)) return PKV_EUNSUPPORTED;
  if (is16(cache_dtype) && cache_dtype != q_dtype) return PKV_EINVAL;
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_context_len < 0)
    return PKV_EINVAL;
  if (batch > kMaxBatch) return PKV_EUNSUPPORTED;
  if (num_q_heads % num_kv_heads) return PKV_EINVAL;
  const int group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return PKV_EUNSUPPORTED;
  int st = check_head_dim(head_dim);
  if (st != PKV_OK) return st;
  st = check_block_size(block_size);
  if (st != PKV_OK) return st;
  if (partition_size < 0 || partition_size % 16) return PKV_EINVAL;
  if (partition_size > kMaxPartition) return PKV_EUNSUPPORTED;
  if (!std::isfinite(sm_scale)) return PKV_EINVAL;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_EINVAL;
  if (q_stride_b < 0 || q_stride_h < 0 || o_stride_b < 0 || o_stride_h < 0 ||
      c_stride_block < 0 || c_stride_slot < 0 || c_stride_head < 0)
    return PKV_EINVAL;
  if (!aligned(q, 16) || !aligned(out, 16) || q_stride_b % 8 || q_stride_h % 8 ||
      o_stride_b % 8 || o_stride_h % 8)
    return PKV_EINVAL;
  CacheKind kind = CacheKind::Same;
  if (cache_dtype == PKV_U3) {
    kind = CacheKind::U3;
    if (!aligned(k_cache, 4) || !aligned(v_cache, 4)) return PKV_EINVAL;
    if (!k_meta || !v_meta || !aligned(k_meta, 4) || !aligned(v_meta, 4)) return PKV_EINVAL;
  } else if (is_byte_code(cache_dtype)) {
    // one lane reads 8 codes (8 bytes) of a row; one fp32 scale per (slot, kv head)
    kind = byte_cache_kind(cache_dtype);
    if (!aligned(k_cache, 8) || !aligned(v_cache, 8) || c_stride_block % 8 || c_stride_slot % 8 ||
        c_stride_head % 8)
      return PKV_EINVAL;
    if (!k_meta || !v_meta || !aligned(k_meta, 4) || !aligned(v_meta, 4)) return PKV_EINVAL;
  } else {
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || c_stride_block % 8 ||
        c_stride_slot % 8 || c_stride_head % 8)
      return PKV_EINVAL;
  }
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4)) return PKV_EINVAL;
  // per-lane row offsets inside a 16-slot chunk are 32-bit byte offsets
  if ((c_stride_slot * 16 + c_stride_head * (int64_t)num_kv_heads) * 4 >= 0x7fffffffLL ||
      (m_ss * 16 + m_sh * (int64_t)num_kv_heads) * 4 >= 0x7fffffffLL)
    return PKV_EUNSUPPORTED;
  if (bt_stride_b < cdiv(max_context_len, block_size)) return PKV_EINVAL;
  const int ps = resolve_partition(partition_size, max_context_len, batch, num_q_heads);
  // granule counts and indices stay in 32 bits
  if ((int64_t)batch * num_kv_heads * cdiv(max_context_len, ps) > 0x7fffffffLL) return PKV_EUNSUPPORTED;
  if (batch == 0) return PKV_OK;
  const DecodeLayout L = decode_layout(batch, num_q_heads, num_kv_heads, head_dim, max_context_len, ps,
                                       q_dtype == PKV_BF16 ? 1 : 0, static_cast<int>(kind));
  if (!workspace || workspace_bytes < L.bytes || !aligned(workspace, 256)) return PKV_EWORKSPACE;

  pkv::DecodeParams p{};
  p.out = out;
  p.q = q;
  p.q_sb = q_stride_b;
  p.q_sh = q_stride_h;
  p.o_sb = o_stride_b;
  p.o_sh = o_stride_h;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.c_sb = c_stride_block;
  p.c_ss = c_stride_slot;
  p.c_sh = c_stride_head;
  p.k_meta = k_meta;
  p.v_meta = v_meta;
  p.m_sb = m_sb;
  p.m_ss = m_ss;
  p.m_sh = m_sh;
  p.block_tables = block_tables;
  p.bt_sb = bt_stride_b;
  p.context_lens = context_lens;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.batch = batch;
  p.block_size = block_size;
  p.log2_bs = log2_exact(block_size);
  p.num_blocks = num_blocks;
  p.max_context_len = max_context_len;
  p.partition_size = ps;
  p.num_wgs = L.plan.num_wgs;
  p.split_tier = L.plan.split_tier;
  p.seg_start_units =
      ((is_byte_code(cache_dtype) || cache_dtype == PKV_U3 ? kSegmentStartTokensCoded : kSegmentStartTokens) + ps / 2) / ps;
  p.heads_per_group = L.plan.heads_per_group;
  p.num_head_groups = L.plan.num_head_groups;
  p.token_streams = L.plan.token_streams;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.u3_code_mask = 0x03800380u;
  p.u3_code_bias = 0x48004800u;
  char* ws = static_cast<char*>(workspace);
  p.ws_acc = reinterpret_cast<float*>(ws + L.acc_off);
  p.ws_ml = reinterpret_cast<float*>(ws + L.ml_off);
  p.ws_seg = reinterpret_cast<int*>(ws + L.seg_off);
  if (nr) {
    p.k_new = nr->k;
    p.v_new = nr->v;
    p.kn_sb = nr->k_sb;
    p.kn_sh = nr->k_sh;
    p.vn_sb = nr->v_sb;
    p.vn_sh = nr->v_sh;
  }
  const SplitWeights sw = cache_dtype == PKV_U3 ? kSplitStaticU3 : kSplitStatic;
  p.split_w[0] = sw.first_even;
  p.split_w[1] = sw.first_odd;
  p.split_w[2] = sw.rest_even;
  p.split_w[3] = sw.rest_odd;
  const hipError_t e = pkv::launch_decode(p, L.plan, kind, q_dtype == PKV_BF16, head_dim, group, stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

int paged_decode(void* out, const void* q, pkv_dtype q_dtype,
                 int64_t q_stride_b, int64_t q_stride_h, int64_t o_stride_b, int64_t o_stride_h,
                 const void* k_cache, const void* v_cache, pkv_dtype cache_dtype,
                 int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                 const void* k_meta, const void* v_meta,
                 const int32_t* block_tables, int64_t bt_stride_b, const int32_t* context_lens,
                 int batch, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                 int64_t num_blocks, int max_context_len, float sm_scale, int partition_size,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // one meta entry per row, [num_blocks, block_size, num_kv_heads]
  return decode_impl(out, q, q_dtype, q_stride_b, q_stride_h, o_stride_b, o_stride_h, k_cache, v_cache,
                     cache_dtype, c_stride_block, c_stride_slot, c_stride_head, k_meta, v_meta,
                     block_tables, bt_stride_b, context_lens, batch, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_context_len, sm_scale, partition_size,
                     workspace, workspace_bytes, stream, (int64_t)block_size * num_kv_heads,
                     num_kv_heads, 1);
}

int paged_decode_scaled(void* out, const void* q, pkv_dtype q_dtype,
                        int64_t q_stride_b, int64_t q_stride_h, int64_t o_stride_b, int64_t o_stride_h,
                        const void* k_cache, const void* v_cache, pkv_dtype cache_dtype,
                        int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                        const float* k_scale, const float* v_scale,
                        int64_t s_stride_block, int64_t s_stride_slot, int64_t s_stride_head,
                        const int32_t* block_tables, int64_t bt_stride_b, const int32_t* context_lens,
                        int batch, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                        int64_t num_blocks, int max_context_len, float sm_scale, int partition_size,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!is_byte_code(cache_dtype)) return PKV_EINVAL;
  return decode_impl(out, q, q_dtype, q_stride_b, q_stride_h, o_stride_b, o_stride_h, k_cache, v_cache,
                     cache_dtype, c_stride_block, c_stride_slot, c_stride_head, k_scale, v_scale,
                     block_tables, bt_stride_b, context_lens, batch, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_context_len, sm_scale, partition_size,
                     workspace, workspace_bytes, stream, s_stride_block, s_stride_slot, s_stride_head);
}

int paged_decode_append(void* out, const void* q, pkv_dtype q_dtype,
                        int64_t q_stride_b, int64_t q_stride_h, int64_t o_stride_b, int64_t o_stride_h,
                        const void* k_new, const void* v_new, int64_t k_new_stride_b, int64_t k_new_stride_h,
                        int64_t v_new_stride_b, int64_t v_new_stride_h,
                        void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                        int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                        void* k_meta, void* v_meta,
                        const int32_t* block_tables, int64_t bt_stride_b, const int32_t* context_lens,
                        int batch, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                        int64_t num_blocks, int max_context_len, float sm_scale, int partition_size,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const NewRows nr{k_new, v_new, k_new_stride_b, k_new_stride_h, v_new_stride_b, v_new_stride_h};
  return decode_impl(out, q, q_dtype, q_stride_b, q_stride_h, o_stride_b, o_stride_h, k_cache, v_cache,
                     cache_dtype, c_stride_block, c_stride_slot, c_stride_head, k_meta, v_meta,
                     block_tables, bt_stride_b, context_lens, batch, num_q_heads, num_kv_heads,
                     head_dim, block_size, num_blocks, max_context_len, sm_scale, partition_size,
                     workspace, workspace_bytes, stream, (int64_t)block_size * num_kv_heads,
                     num_kv_heads, 1, &nr);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// paged_decode_noalloc: paged_decode with its workspace in a file-scope device array, for callers
// that cannot allocate.  `scratch` is a host-side stand-in for the array in host code; its device
// address, which differs per GPU, comes from hipGetSymbolAddress on each device's first call and
// is the only form in which host code passes the array on.
// ---------------------------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t(24) << 20;          // 24 MiB per GPU
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up once per device, with that device current).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PKV_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}
}  // namespace

extern "C" int paged_decode_noalloc(void* out, const void* q, pkv_dtype q_dtype,
                                    int64_t q_stride_b, int64_t q_stride_h, int64_t o_stride_b,
                                    int64_t o_stride_h, const void* k_cache, const void* v_cache,
                                    pkv_dtype cache_dtype, int64_t c_stride_block, int64_t c_stride_slot,
                                    int64_t c_stride_head, const void* k_meta, const void* v_meta,
                                    const int32_t* block_tables, int64_t bt_stride_b,
                                    const int32_t* context_lens, int batch, int num_q_heads,
                                    int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                                    int max_context_len, float sm_scale, int partition_size,
                                    hipStream_t stream) {
  void* ws = nullptr;
  const int st = scratch_of_current_device(&ws);
  if (st != PKV_OK) return st;
  // the same validation and kernels as paged_decode; the only workspace error left is a call
  // whose partial states do not fit the static buffer
  const int r = decode_impl(out, q, q_dtype, q_stride_b, q_stride_h, o_stride_b, o_stride_h, k_cache,
                            v_cache, cache_dtype, c_stride_block, c_stride_slot, c_stride_head, k_meta,
                            v_meta, block_tables, bt_stride_b, context_lens, batch, num_q_heads,
                            num_kv_heads, head_dim, block_size, num_blocks, max_context_len, sm_scale,
                            partition_size, ws, kScratchBytes, stream, (int64_t)block_size * num_kv_heads,
                            num_kv_heads, 1);
  return r == PKV_EWORKSPACE ? PKV_ESCRATCH : r;
}

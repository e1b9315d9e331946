/*
 * pagedkv.h - C ABI of the paged KV-cache hot path for AMD MI355X (gfx950).
 *
 * Pages the operations are defined by:
 *   [Append] "Write Triton Kv Cache Append Kernel" (skillsdirectory.com skill page)
 *   [Paged]  "Triton KV Cache and PagedAttention" (datawhalechina llm-algo-leetcode, ch. 10)
 *   [3bit]   "triton-3bit-kv-cache-kernel" (GitHub README)
 *
 * General contract (every entry point):
 *   - Every buffer is owned by the caller.  The library never allocates or frees
 *     memory and keeps no state between calls.  Device pointers must point to
 *     memory of the current HIP device.
 *   - Work is enqueued on `stream` and is asynchronous; ordering against other
 *     streams, and against host-side updates of block tables or slot mappings,
 *     is the caller's job (same stream => ordered).  [Append], Common failure modes.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     negative return value means nothing was enqueued and nothing was written:
 *       PKV_EINVAL        malformed argument (null pointer, bad size or stride,
 *                         misaligned pointer, Hq not a multiple of Hkv, ...)
 *       PKV_EUNSUPPORTED  well-formed but outside the compiled set (head_dim not
 *                         64/128, block_size not 16/32/64, group size not 1/2/4/8,
 *                         dtype combination not provided)
 *       PKV_EWORKSPACE    workspace missing or smaller than required
 *       PKV_EHIP          the kernel launch itself failed (hipGetLastError)
 *   - Strides are in ELEMENTS of the tensor's own element type (uint32 words for a
 *     3-bit cache), never bytes.  The innermost (head_dim) stride is always 1.
 *   - Grids depend only on the shape arguments (and max_context_len), never on
 *     the contents of slot_mapping / context_lens, so calls can be captured in a
 *     HIP graph at a padded maximum batch.  [Append], Performance requirements.
 *   - Calls that share an output buffer (or a decode workspace) on different
 *     streams without ordering race.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,
  PKV_EUNSUPPORTED = -2,
  PKV_EWORKSPACE = -3,
  PKV_EHIP = -4,
  PKV_ESCRATCH = -5    /* paged_decode_noalloc: the call needs more than its static scratch */
} pkv_status;

typedef enum {
  PKV_F16 = 0,         /* IEEE binary16                                             */
  PKV_BF16 = 1,        /* bfloat16                                                  */
  PKV_FP8_E4M3FN = 2,  /* OCP FP8 E4M3 (finite-only, max 448), one fp32 scale per row */
  PKV_U3 = 3,          /* 3-bit affine codes, 32 per 3 uint32 words, fp16 (scale, zero) per row */
  PKV_FP8_E5M2 = 4,    /* OCP FP8 E5M2 (bias 15, max finite 57344), one fp32 scale per row  */
  PKV_INT8 = 5         /* signed 8-bit integers in [-127, 127], one fp32 scale per row      */
} pkv_dtype;

/*
 * kv_append - write new K and V rows into a paged block pool through slot_mapping.
 *
 * Defined by [Append], Required reasoning process steps 1-8 (unified prefill and
 * decode interface; slot = block_id * block_size + slot_in_block; slot < 0 is a
 * no-op taken before any load; K and V in one pass; scale division in fp32 before
 * the cast), Inputs items 1-9, Kernel design rules; the fp8 e4m3 / e5m2 and int8 caches
 * by [Append], Inputs item 4 and step 6; the packed 3-bit cache by [3bit], sections 1A/1B
 * (bit layout) and 2, test 3 (fp16 affine scale/zero).
 *
 *   k_new, v_new     device, [num_tokens, num_kv_heads, head_dim] of in_dtype (F16
 *                    or BF16); element (t, h, d) at t*stride_tok + h*stride_head + d.
 *                    Rows must be 16-byte aligned (pointer and both strides).  May
 *                    be views into a fused QKV buffer.
 *   slot_mapping     device int64 [num_tokens].  slot < 0: padding, nothing of token
 *                    t is read or written.  slot >= num_blocks*block_size: skipped
 *                    (a caller error, handled defensively).  Two tokens with the same
 *                    slot in one call: undefined which one wins.
 *   k_cache, v_cache device pools [num_blocks, block_size, num_kv_heads, R] where R is
 *                    head_dim elements (F16/BF16, or bytes for FP8/INT8) or head_dim*3/32 uint32 words
 *                    (U3); row (blk, slot, h) at blk*c_stride_block +
 *                    c_stride_slot*slot + c_stride_head*h.  16-byte aligned rows
 *                    (8-byte for U3 with head_dim 64).  Any strides of that form are
 *                    accepted, e.g. the dual-stacked block layout [num_blocks, 2,
 *                    num_kv_heads, block_size, head_dim] as two views (k_cache = base,
 *                    v_cache = base + num_kv_heads*block_size*head_dim, c_stride_block =
 *                    2*num_kv_heads*block_size*head_dim, c_stride_slot = head_dim,
 *                    c_stride_head = block_size*head_dim); k_cache and v_cache share the
 *                    strides.  The contiguous cache [batch, num_kv_heads, max_seq_len,
 *                    head_dim] with slot = request*max_seq_len + position ([Append] step 5)
 *                    is the pool whose block is one request: num_blocks = batch, block_size =
 *                    max_seq_len (a power of two), c_stride_block = num_kv_heads*max_seq_len*
 *                    head_dim, c_stride_slot = head_dim, c_stride_head = max_seq_len*head_dim.
 *   cache_dtype      == in_dtype (bit copy), or PKV_FP8_E4M3FN, PKV_FP8_E5M2, PKV_INT8
 *                    (the byte-code caches: pools 8-byte aligned, strides multiples of 8),
 *                    or PKV_U3.
 *   k_meta, v_meta   byte-code caches: fp32 [num_blocks, block_size, num_kv_heads] per-row
 *                    scales s = absmax/M with M = 448 (E4M3FN), 57344 (E5M2) or 127
 *                    (INT8), s = 1 for an all-zero row; y = clamp(x/s, +-M) with the
 *                    correctly rounded fp32 quotient; code = RNE_e4m3fn(y), RNE_e5m2(y) or
 *                    rint(y) (ties to even).  U3: fp16 [num_blocks, block_size,
 *                    num_kv_heads, 2] = (s, z), per-row min/max affine parameters
 *                    (s = fp16((max-min)/7), z = fp16(-min/s), q = clamp(rint(x/s+z),
 *                    0, 7); degenerate rows use s = 1, z = fp16(-min)).  Contiguous.
 *                    NULL for same-dtype caches.
 *   head_dim         64 or 128.   block_size a power of two from 16 to 2^24 (paged_decode
 *                    reads pools of 16, 32 or 64).   num_tokens >= 0, and
 *                    num_tokens * num_kv_heads < 2^31 (else PKV_EUNSUPPORTED).
 * Inputs must be finite for the quantised caches.  Bit-exact by contract.
 */
int kv_append(const void* k_new, const void* v_new, pkv_dtype in_dtype,
              int64_t k_stride_tok, int64_t k_stride_head,
              int64_t v_stride_tok, int64_t v_stride_head,
              const int64_t* slot_mapping, int64_t num_tokens,
              void* k_cache, void* v_cache, pkv_dtype cache_dtype,
              int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
              void* k_meta, void* v_meta,
              int64_t num_blocks, int block_size, int num_kv_heads, int head_dim,
              hipStream_t stream);

/*
 * kv_append_scaled - kv_append into a byte-code cache with scales the caller supplies.
 *
 * Defined by [Append], Inputs items 4 and 8 (fp8 / int8 caches with fp32 scales of per-tensor,
 * per-token, per-head or per-block granularity, and their shape and indexing) and Required
 * reasoning process step 6 (a per-tensor scale is divided out before the cast; per-token or
 * per-block scales are loaded first).  Arguments as for kv_append, except:
 *   cache_dtype      PKV_FP8_E4M3FN, PKV_FP8_E5M2 or PKV_INT8 (else PKV_EINVAL).
 *   k_scale, v_scale device fp32, read only: the scale of row (blk, slot, h) is
 *                    scale[blk*s_stride_block + slot*s_stride_slot + h*s_stride_head]
 *                    (strides >= 0, in floats).  Per tensor: (0, 0, 0); per head: (0, 0, 1);
 *                    per block: (1, 0, 0); per block and head: (num_kv_heads, 0, 1); per token
 *                    and head: (block_size*num_kv_heads, num_kv_heads, 1).  Scales must be
 *                    positive and finite (not checked: other values give undefined codes).
 * Codes: y = clamp(x/s, +-M) with the correctly rounded fp32 quotient, M = 448, 57344 or 127,
 * then RNE_e4m3fn(y), RNE_e5m2(y) or rint(y) (ties to even).  The scales are never written.
 * Bit-exact by contract.
 */
int kv_append_scaled(const void* k_new, const void* v_new, pkv_dtype in_dtype,
                     int64_t k_stride_tok, int64_t k_stride_head,
                     int64_t v_stride_tok, int64_t v_stride_head,
                     const int64_t* slot_mapping, int64_t num_tokens,
                     void* k_cache, void* v_cache, pkv_dtype cache_dtype,
                     int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                     const float* k_scale, const float* v_scale,
                     int64_t s_stride_block, int64_t s_stride_slot, int64_t s_stride_head,
                     int64_t num_blocks, int block_size, int num_kv_heads, int head_dim,
                     hipStream_t stream);

/*
 * paged_decode_workspace_size - bytes of workspace paged_decode needs.
 *
 * Split-K ("flash-decoding", named by [3bit] in its title paragraph as the form of its fused
 * decode): the context of each (request, kv head) may be cut into token ranges that are
 * reduced independently and merged by log-sum-exp.  The library balances the work by
 * giving each resident workgroup of the current device a share of all (request, kv head,
 * granule) units sized to its expected speed, where a granule is `partition_size` tokens;
 * a context is cut at multiples of the granule.  The workspace holds the partial states of
 * the ranges that get cut, so its size depends on the current device's compute-unit count: query it on the
 * device that will run the call.
 * partition_size: 0 = automatic (16 tokens, the finest balance), else a multiple of 16.
 * Returns 0 for batch 0 and (size_t)-1 for invalid arguments (batch above 8192 included).
 */
size_t paged_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                   int max_context_len, int partition_size);

/*
 * paged_decode - single-query attention over a paged KV cache (one decode step).
 *
 * Defined by [Paged], Step 1 and the reference answer (TODO 1-5): for request b and
 * query head h, out[b,h] = sum_t softmax_t(sm_scale * q[b,h].k_t) v_t over the first
 * context_lens[b] tokens, token t read from physical block block_tables[b, t /
 * block_size] at slot t % block_size; GQA per [Append] (query head h reads kv head
 * h / (num_q_heads / num_kv_heads)); with the 3-bit cache the codes are unpacked and
 * dequantised, x = (q - z) * s, on the fly ([3bit], title paragraph, section 2 test 3);
 * with a byte-code cache (fp8 e4m3fn, fp8 e5m2, int8) each row reads as decode(code) * s,
 * the inverse of the kv_append quantiser ([Append], Inputs item 4 and Correctness
 * requirements: the quantised cache is read back through the row's scale), with s applied to
 * the row's dot product and to its probability.
 *
 *   out, q           device [batch, num_q_heads, head_dim] of q_dtype (F16 or BF16);
 *                    element (b, h, d) at b*stride_b + h*stride_h + d; out has the
 *                    same dtype.  16-byte aligned rows.
 *   k_cache, v_cache pools as for kv_append; cache_dtype == q_dtype, or PKV_U3 (with
 *                    k_meta, v_meta fp16 (s, z) as for kv_append), or PKV_FP8_E4M3FN,
 *                    PKV_FP8_E5M2 or PKV_INT8 (with k_meta, v_meta fp32 per-row scales as
 *                    for kv_append; pools 8-byte aligned, strides multiples of 8, else
 *                    PKV_EINVAL).
 *   block_tables     device int32 [batch, bt_stride_b >= cdiv(max_context_len,
 *                    block_size)]; entries at or beyond cdiv(context_lens[b],
 *                    block_size) are never read.  Entries must be < num_blocks.
 *   context_lens     device int32 [batch], 0 <= context_lens[b] <= max_context_len.
 *                    context_lens[b] == 0 gives an all-zero output row.
 *   sm_scale         score scale (the pages use 1/sqrt(head_dim)).
 *   partition_size   split granule in tokens (0 = automatic; else a multiple of 16); see
 *                    paged_decode_workspace_size.
 *   workspace        device, >= paged_decode_workspace_size(...) bytes, 256-byte aligned,
 *                    with any contents: a call reads nothing from it that the same call did
 *                    not write first, so a fresh uninitialised allocation is fine and one workspace serves calls of every shape it is
 *                    large enough for.  Calls sharing a workspace must be ordered (same
 *                    stream, or synchronised); overlapping calls on it race.
 *   batch            0 .. 8192.
 * Accumulation is fp32; outputs are rounded to q_dtype to nearest even.
 * Reproducibility: results are fixed up to the order of the fp32 additions.  The token streams
 * of a workgroup share a range's chunks at run time, so which wave sums which tokens, and in
 * which order, depends on timing (which workgroup reads which tokens does not: the split over
 * workgroups is fixed by the context lengths and the partition size).  Two calls on the same inputs attend over the same tokens with the same weights and
 * agree to within fp32 rounding of the sums (far inside the 2e-3 attention tolerance), not bit
 * for bit.
 */
int paged_decode(void* out, const void* q, pkv_dtype q_dtype,
                 int64_t q_stride_b, int64_t q_stride_h, int64_t o_stride_b, int64_t o_stride_h,
                 const void* k_cache, const void* v_cache, pkv_dtype cache_dtype,
                 int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                 const void* k_meta, const void* v_meta,
                 const int32_t* block_tables, int64_t bt_stride_b, const int32_t* context_lens,
                 int batch, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                 int64_t num_blocks, int max_context_len, float sm_scale, int partition_size,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_decode_scaled - paged_decode over a byte-code cache whose scales the caller supplies
 * (the cache kv_append_scaled writes).
 *
 * Defined as paged_decode ([Paged], Step 1 and TODO 1-5), with each row read as decode(code) *
 * s and s found as in kv_append_scaled ([Append], Inputs items 4 and 8: scale granularity and
 * indexing).  Arguments as for paged_decode, except:
 *   cache_dtype      PKV_FP8_E4M3FN, PKV_FP8_E5M2 or PKV_INT8 (else PKV_EINVAL).
 *   k_scale, v_scale device fp32, read only, row (blk, slot, h) at blk*s_stride_block +
 *                    slot*s_stride_slot + h*s_stride_head (strides >= 0, in floats;
 *                    (16*s_stride_slot + num_kv_heads*s_stride_head)*4 < 2^31, else
 *                    PKV_EUNSUPPORTED).
 * The workspace is shared with paged_decode (same size query).
 */
int paged_decode_scaled(void* out, const void* q, pkv_dtype q_dtype,
                        int64_t q_stride_b, int64_t q_stride_h, int64_t o_stride_b, int64_t o_stride_h,
                        const void* k_cache, const void* v_cache, pkv_dtype cache_dtype,
                        int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                        const float* k_scale, const float* v_scale,
                        int64_t s_stride_block, int64_t s_stride_slot, int64_t s_stride_head,
                        const int32_t* block_tables, int64_t bt_stride_b, const int32_t* context_lens,
                        int batch, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                        int64_t num_blocks, int max_context_len, float sm_scale, int partition_size,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_decode_append - one decode step in one launch: the new token of every request is
 * appended to the cache, then the decode attends over the cache including it.
 *
 * Defined as kv_append of k_new / v_new ([Append], Required reasoning process steps 1-9) with
 * request b's token at slot block_tables[b, pos / block_size] * block_size + pos % block_size,
 * pos = context_lens[b] - 1 (the slot construction of step 9 for a decode token; no token for a
 * request with context_lens[b] == 0), followed by paged_decode ([Paged], Step 1 and TODO 1-5)
 * with the same context_lens: the same pool contents (bit for bit) and the same outputs as those
 * two calls.  The workgroup of the decode that reads a request's last token writes that token
 * first, so nothing else is launched for the append.
 *   k_new, v_new     device [batch, num_kv_heads, head_dim] of q_dtype, element (b, h, d) at
 *                    b*stride_b + h*stride_h + d (strides >= 0, multiples of 8; 16-byte
 *                    aligned), read only.
 *   k_cache, v_cache, k_meta, v_meta  as for kv_append (written: the new rows, and for the
 *                    quantised caches their per-row scales or (s, z) pairs, computed as kv_append
 *                    computes them) and for paged_decode (read).
 *   other arguments  as for paged_decode.  The context lengths count the new token.
 * A block id outside [0, num_blocks) skips that request's write, as kv_append skips a slot
 * outside the pool.  The workspace is shared with paged_decode (same size query).
 */
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
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_decode_noalloc - paged_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Arguments, validation, kernels and results as for paged_decode, without workspace arguments:
 * the partial states go to a static device array of 24 MiB that the library holds on each GPU
 * it runs on until the process ends (its device address is looked up on the first call on each
 * device).  The call allocates and frees nothing.  Limit: a call whose workspace
 * (paged_decode_workspace_size of its shape, on this device) exceeds 24 MiB returns
 * PKV_ESCRATCH and writes nothing; on a 256-CU MI355X the long-context shape (batch 8, 64 / 8
 * heads, head_dim 128) needs about 16.3 MiB and the Llama-8B decode shape about 8.5 MiB.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (different streams without ordering, or
 * several threads) race and give undefined results; ordered calls are independent (each call
 * writes what it reads).
 */
int paged_decode_noalloc(void* out, const void* q, pkv_dtype q_dtype,
                         int64_t q_stride_b, int64_t q_stride_h, int64_t o_stride_b, int64_t o_stride_h,
                         const void* k_cache, const void* v_cache, pkv_dtype cache_dtype,
                         int64_t c_stride_block, int64_t c_stride_slot, int64_t c_stride_head,
                         const void* k_meta, const void* v_meta,
                         const int32_t* block_tables, int64_t bt_stride_b, const int32_t* context_lens,
                         int batch, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                         int64_t num_blocks, int max_context_len, float sm_scale, int partition_size,
                         hipStream_t stream);

/*
 * build_slot_mapping - the slot id of every new token from its request and position.
 *
 * Defined by [Append], Inputs items 6 and 7 and Required reasoning process step 9 (the
 * launcher's step: paged slot = block_id * block_size + slot_in_block with the physical block
 * of the token's logical block; a decode token's position is the context length before the
 * increment).
 *   token_request    device int32 [num_tokens], or NULL: token t belongs to request t (one
 *                    decode token per request).  A negative entry marks a padding token.
 *   token_position   device int32 [num_tokens], the token's position in its sequence.
 *   block_tables     device int32 [batch, bt_stride_b] (bt_stride_b >= 1): slot =
 *                    block_tables[r, p / block_size] * block_size + p % block_size.  NULL: the
 *                    contiguous cache, slot = r * block_size + p with block_size = max_seq_len.
 *   block_size       a power of two from 16 to 2^24.
 *   slot_mapping     device int64 [num_tokens], written.  -1 where the request is negative or
 *                    >= batch, or the position is negative, outside the table row (p /
 *                    block_size >= bt_stride_b) or, without a table, >= block_size: kv_append
 *                    then skips the token.
 * num_tokens < 2^31.  Bit-exact.  Entries of the table row beyond the position's block are not read.
 */
int build_slot_mapping(const int32_t* token_request, const int32_t* token_position, int64_t num_tokens,
                       const int32_t* block_tables, int64_t bt_stride_b, int batch, int block_size,
                       int64_t* slot_mapping, hipStream_t stream);

/*
 * pack3 / unpack3 - 3-bit packing, [3bit] sections 1A and 1B: value j of each group
 * of 8 sits at bits 3j..3j+2 of a 24-bit little-endian octet (3 bytes); 32 values
 * therefore fill 3 little-endian uint32 words with lane i at bit 3i.
 *   pack3:   values  device uint8 [n_values] (only the low 3 bits are used)
 *            -> packed device uint8 [3*n_values/8].
 *   unpack3: packed  device uint8 [3*n_values/8] -> values device uint8 [n_values],
 *            each in 0..7.
 * n_values >= 0 and a multiple of 8.  No alignment requirement.  Bit-exact.
 */
int pack3(const uint8_t* values, uint8_t* packed, int64_t n_values, hipStream_t stream);
int unpack3(const uint8_t* packed, uint8_t* values, int64_t n_values, hipStream_t stream);

/* Human-readable text for a pkv_status value (static storage; never NULL). */
const char* pkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */

"""CPU oracle for the paged KV-cache path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg do.  It is plain numpy, written from the pages'
definitions, and shares no code with the HIP library (no kernels, headers,
helpers, tables or pre/post-processing); the only module both sides consume
is the seeded input generator, which holds none of the method's arithmetic.

Pages cited throughout (each module repeats the titles it uses):
  [Append]  "Write Triton Kv Cache Append Kernel" (skillsdirectory.com skill page)
  [Paged]   "Triton KV Cache and PagedAttention" (datawhalechina llm-algo-leetcode, ch. 10)
  [3bit]    "triton-3bit-kv-cache-kernel" (GitHub README)

Precision: attention runs in float64; the fp8 and 3-bit quantisers run in
float32 with the operation order stated in each function, because the append
page requires the scale division in fp32 and bit-exact parity needs the same
fp32 sequence on both sides.

Pin status of every function is listed in its docstring ("pinned by" ...).
"""
from .pack3 import (pack3, unpack3, pack3_words, unpack3_words, pack_rows_u3,
                    unpack_rows_u3)
from .fp8 import (e4m3fn_decode_table, e4m3fn_encode_rne, e4m3fn_decode,
                  quantize_fp8_rows, dequantize_fp8_rows, E4M3_MAX)
from .quant3 import quantize_u3_rows, dequantize_u3_rows
from .quant8 import (e5m2_decode_table, e5m2_decode, e5m2_encode_rne, quantize_e5m2_rows,
                     quantize_int8_rows, dequantize_e5m2_rows, dequantize_int8_rows, E5M2_MAX,
                     INT8_MAX, quantize_given_scale, scale_offsets)
from .slots import decode_slot_mapping, prefill_slot_mapping, slot_mapping_ref
from .append import append_ref, CacheSpec
from .attention import (paged_decode_ref, paged_decode_split_ref, lse_merge_ref,
                        gather_rows_f64, PoolView)

__all__ = [
    "pack3", "unpack3", "pack3_words", "unpack3_words", "pack_rows_u3", "unpack_rows_u3",
    "e4m3fn_decode_table", "e4m3fn_encode_rne", "e4m3fn_decode", "quantize_fp8_rows",
    "dequantize_fp8_rows", "E4M3_MAX", "quantize_u3_rows", "dequantize_u3_rows",
    "e5m2_decode_table", "e5m2_decode", "e5m2_encode_rne", "quantize_e5m2_rows",
    "quantize_int8_rows", "dequantize_e5m2_rows", "dequantize_int8_rows", "E5M2_MAX", "INT8_MAX",
    "quantize_given_scale", "scale_offsets",
    "decode_slot_mapping", "prefill_slot_mapping", "slot_mapping_ref", "append_ref", "CacheSpec",
    "paged_decode_ref", "paged_decode_split_ref", "lse_merge_ref", "gather_rows_f64", "PoolView",
]

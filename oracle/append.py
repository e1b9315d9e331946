"""KV append oracle (test infrastructure only).

Pages cited: [Append] "Write Triton Kv Cache Append Kernel" (skillsdirectory.com),
  * Inputs the agent should gather first, items 1, 3, 5, 6, 9 (paged layout
    [num_blocks, block_size, num_kv_heads, head_dim]; the cache holds only the
    kv heads; new K/V [num_tokens, num_kv_heads, head_dim] with arbitrary strides),
  * Required reasoning process, steps 3-8 (slot < 0 is a no-op taken before any
    load; block = slot // block_size, offset = slot % block_size; quantise after
    scaling; K and V handled together),
  * Correctness requirements (exactly one slot per token; pure write; idempotence).
  [3bit] "triton-3bit-kv-cache-kernel" (GitHub README), title paragraph and
  sections 1 and 2 (the packed 3-bit cache with fp16 scale/zero).

Cache element types:
  "same"  - the cache has the input's dtype; the row is copied bit for bit,
  "fp8"   - e4m3fn codes, with one fp32 scale per (block, slot, kv head),
  "e5m2"  - e5m2 codes, scaled the same way (oracle/quant8.py),
  "i8"    - int8 codes (stored as their bytes), scaled the same way (oracle/quant8.py),
  "u3"    - 3-bit codes packed 32 per 3 uint32 words (head_dim*3/32 words per
            row), with an fp16 (scale, zero) pair per (block, slot, kv head).

Out-of-range slots (slot >= num_blocks * block_size) are skipped like padding:
the pages assume valid slots, and skipping is the defensive reading.

Pinned by: readback through the slot ids, whole-pool equality against an
untouched copy outside the written slots, idempotence, and the quantiser pins.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .fp8 import quantize_fp8_rows
from .quant8 import quantize_e5m2_rows, quantize_int8_rows, quantize_given_scale, scale_offsets
from .quant3 import quantize_u3_rows
from .pack3 import pack_rows_u3


@dataclasses.dataclass
class CacheSpec:
    kind: str                 # "same" | "fp8" | "e5m2" | "i8" | "u3"
    in_dtype: str             # "f16" | "bf16"


def to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 bit patterns of fp16/bf16 values -> exact float32 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def append_ref(k_new_bits: np.ndarray, v_new_bits: np.ndarray, slot_mapping: np.ndarray,
               k_cache: np.ndarray, v_cache: np.ndarray, spec: CacheSpec, block_size: int,
               k_meta: Optional[np.ndarray] = None, v_meta: Optional[np.ndarray] = None,
               scale_strides=None) -> None:
    """Update the caches in place.

    k_new_bits, v_new_bits: uint16 [T, Hkv, D] (the raw fp16/bf16 bits).
    k_cache, v_cache: "same": uint16 [NB, BS, Hkv, D]; "fp8", "e5m2", "i8": uint8 [NB, BS, Hkv, D];
                      "u3": uint32 [NB, BS, Hkv, 3*D/32].
    k_meta, v_meta:   "fp8", "e5m2", "i8": float32 [NB, BS, Hkv]; "u3": float16 [NB, BS, Hkv, 2].
    scale_strides:    byte-code caches only: None = the append computes and writes one scale
                      per row (above); (sb, ss, sh) = k_meta / v_meta are the caller's scale
                      arrays (any shape, read flat at block*sb + slot*ss + head*sh) and are
                      only read (oracle/quant8.py, caller-given scales).
    """
    nb = k_cache.shape[0]
    T = slot_mapping.shape[0]
    for t in range(T):
        slot = int(slot_mapping[t])
        if slot < 0 or slot >= nb * block_size:
            continue                      # no-op, and nothing of token t is read
        blk, off = divmod(slot, block_size)
        for src, cache, meta in ((k_new_bits, k_cache, k_meta), (v_new_bits, v_cache, v_meta)):
            row_bits = np.asarray(src[t])                 # [Hkv, D]
            if spec.kind == "same":
                cache[blk, off] = row_bits
            elif scale_strides is not None and spec.kind in ("fp8", "e5m2", "i8"):
                heads = np.arange(row_bits.shape[0])
                s = meta.reshape(-1)[scale_offsets(blk, off, heads, scale_strides)]
                cache[blk, off] = quantize_given_scale(to_f32(row_bits, spec.in_dtype), s, spec.kind)
            elif spec.kind == "fp8":
                codes, scale = quantize_fp8_rows(to_f32(row_bits, spec.in_dtype))
                cache[blk, off] = codes
                meta[blk, off] = scale
            elif spec.kind in ("e5m2", "i8"):
                quant = quantize_e5m2_rows if spec.kind == "e5m2" else quantize_int8_rows
                codes, scale = quant(to_f32(row_bits, spec.in_dtype))
                cache[blk, off] = codes.view(np.uint8)
                meta[blk, off] = scale
            elif spec.kind == "u3":
                q, s16, z16 = quantize_u3_rows(to_f32(row_bits, spec.in_dtype))
                cache[blk, off] = pack_rows_u3(q)
                meta[blk, off, :, 0] = s16
                meta[blk, off, :, 1] = z16
            else:
                raise ValueError(spec.kind)

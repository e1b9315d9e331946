"""Paged decode attention oracle (test infrastructure only), float64.

Pages cited:
  [Paged] "Triton KV Cache and PagedAttention" (datawhalechina llm-algo-leetcode, ch. 10):
    * Step 1 (block pool [num_blocks, block_size, heads, head_dim]; per-request
      block table from logical to physical block; one query token per request),
    * Step 3 and the reference answer, TODO 1-3 (physical block = table entry of
      the logical block; tokens at or beyond the context length are masked out;
      scores are q.k scaled by sm_scale = 1/sqrt(head_dim)),
    * TODO 4-5 and the final normalisation (online softmax, which in exact
      arithmetic equals the plain softmax below).
  [Append] "Write Triton Kv Cache Append Kernel", Inputs item 3 and Kernel design
    rules (GQA: the cache holds num_kv_heads; query heads share kv heads).
  [3bit] "triton-3bit-kv-cache-kernel" README, title paragraph (the fused 3-bit
    flash-decoding reads codes and dequantises them on the fly).

Readings (where the pages leave a step open): q head h reads kv head h // (Hq / Hkv); a request
with context length 0 produces an all-zero output; block-table entries at or
beyond cdiv(L, block_size) are never read; split-K partitions are the token
ranges [P*i, P*(i+1)) counted from token 0, merged by log-sum-exp.

Pinned by: brute-force dense attention (torch's float64 scaled_dot_product_attention
on the block-table-gathered K/V, the construction of the PagedAttention page's own
test), block-permutation invariance, L = 1 -> v_0, equal keys -> mean(V),
GQA == MHA on repeated K/V, NaN-poisoned unused slots not reaching the output, and
(for the split form) equality with the single-pass form to 1e-12.
"""
from __future__ import annotations

import numpy as np

from .append import to_f32
from .fp8 import dequantize_fp8_rows
from .quant8 import dequantize_e5m2_rows, dequantize_int8_rows, scale_offsets
from .pack3 import unpack_rows_u3
from .quant3 import dequantize_u3_rows


class PoolView:
    """A cache pool as the oracle reads it: rows of (block, slot, kv head) -> float64."""

    def __init__(self, kind: str, cache: np.ndarray, meta=None, dtype: str = "bf16",
                 head_dim: int = 0, scale_strides=None):
        self.kind, self.cache, self.meta, self.dtype = kind, cache, meta, dtype
        # byte-code caches with caller-given scales: meta is read flat at
        # block*sb + slot*ss + head*sh (oracle/quant8.py); None = one scale per row
        self.scale_strides = scale_strides
        self.head_dim = head_dim if head_dim else (cache.shape[-1] if kind != "u3"
                                                   else cache.shape[-1] * 32 // 3)

    def rows(self, blocks: np.ndarray, kv_head: int) -> np.ndarray:
        """[n_blocks * BS, D] float64 rows of one kv head, in logical order."""
        c = self.cache[blocks, :, kv_head]                       # [nb, BS, ...]
        if self.scale_strides is not None:
            bs = self.cache.shape[1]
            offs = scale_offsets(np.asarray(blocks)[:, None], np.arange(bs)[None, :], kv_head,
                                 self.scale_strides)
            scales = self.meta.reshape(-1)[offs]
        elif self.kind in ("fp8", "e5m2", "i8"):
            scales = self.meta[blocks, :, kv_head]
        if self.kind == "same":
            out = to_f32(c, self.dtype).astype(np.float64)
        elif self.kind == "fp8":
            out = dequantize_fp8_rows(c, scales)
        elif self.kind == "e5m2":
            out = dequantize_e5m2_rows(c, scales)
        elif self.kind == "i8":
            out = dequantize_int8_rows(c, scales)
        elif self.kind == "u3":
            q = unpack_rows_u3(c, self.head_dim)
            m = self.meta[blocks, :, kv_head]
            out = dequantize_u3_rows(q, m[..., 0], m[..., 1])
        else:
            raise ValueError(self.kind)
        return out.reshape(-1, self.head_dim)


def gather_rows_f64(pool: PoolView, block_table_row: np.ndarray, L: int, block_size: int,
                    kv_head: int) -> np.ndarray:
    """The first L tokens of one request's kv head, through the block table."""
    nblk = -(-L // block_size)
    blocks = np.asarray(block_table_row[:nblk], dtype=np.int64)
    return pool.rows(blocks, kv_head)[:L]


def paged_decode_ref(q: np.ndarray, k_pool: PoolView, v_pool: PoolView, block_tables: np.ndarray,
                     context_lens: np.ndarray, block_size: int, num_kv_heads: int, sm_scale: float,
                     heads=None) -> np.ndarray:
    """q: float [B, Hq, D] -> out float64 [B, Hq, D].

    out[b, h] = sum_t softmax_t(sm_scale * q[b,h] . k_t) v_t over the first
    context_lens[b] tokens of request b, read through block_tables[b].
    `heads` optionally restricts the work to a list of (b, h) pairs (others are 0).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    out = np.zeros((B, Hq, D), dtype=np.float64)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    by_kv = {}
    for b, h in todo:
        by_kv.setdefault((b, h // G), []).append(h)
    for (b, kvh), hs in by_kv.items():
        L = int(context_lens[b])
        if L == 0:
            continue
        K = gather_rows_f64(k_pool, block_tables[b], L, block_size, kvh)
        V = gather_rows_f64(v_pool, block_tables[b], L, block_size, kvh)
        for h in hs:
            s = sm_scale * (K @ q[b, h])
            p = np.exp(s - s.max())
            out[b, h] = (p @ V) / p.sum()
    return out


def lse_merge_ref(m: np.ndarray, l: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """Merge partition states: m [P] running maxima, l [P] sums of exp(s - m_p),
    acc [P, D] sums of exp(s - m_p) v.  Empty partitions have l = 0, m = -inf."""
    m = np.asarray(m, dtype=np.float64)
    live = l > 0
    if not np.any(live):
        return np.zeros(acc.shape[-1], dtype=np.float64)
    M = m[live].max()
    w = np.where(live, np.exp(np.where(live, m - M, 0.0)), 0.0)
    return (w[:, None] * acc).sum(axis=0) / (w * l).sum()


def paged_decode_split_ref(q: np.ndarray, k_pool: PoolView, v_pool: PoolView,
                           block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                           num_kv_heads: int, sm_scale: float, partition_size: int,
                           heads=None) -> np.ndarray:
    """Split-K form: per partition [P*i, P*(i+1)) compute (m_i, l_i, acc_i), then
    merge by log-sum-exp (lse_merge_ref)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    out = np.zeros((B, Hq, D), dtype=np.float64)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        L = int(context_lens[b])
        if L == 0:
            continue
        K = gather_rows_f64(k_pool, block_tables[b], L, block_size, h // G)
        V = gather_rows_f64(v_pool, block_tables[b], L, block_size, h // G)
        nparts = -(-L // partition_size)
        ms, ls, accs = [], [], []
        for i in range(nparts):
            lo, hi = i * partition_size, min(L, (i + 1) * partition_size)
            s = sm_scale * (K[lo:hi] @ q[b, h])
            mi = s.max()
            p = np.exp(s - mi)
            ms.append(mi)
            ls.append(p.sum())
            accs.append(p @ V[lo:hi])
        out[b, h] = lse_merge_ref(np.array(ms), np.array(ls), np.array(accs))
    return out

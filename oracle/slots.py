"""slot_mapping construction oracle (test infrastructure only).

Page cited: [Append] "Write Triton Kv Cache Append Kernel" (skillsdirectory.com),
  * Inputs the agent should gather first, items 6 and 7 (paged slot id =
    block_id * block_size + slot_in_block; block_table maps logical to physical
    blocks),
  * Required reasoning process, step 9 (decode: the new token's position is the
    context length *before* it is incremented; prefill: expand each request's
    positions into per-token slots),
  * Kernel design rules and Common failure modes (slot -1 marks padding; the
    off-by-one and physical-vs-logical block-index mistakes).

Pinned by: agreement with the synthetic allocator's own slot bookkeeping on every
workload, and the off-by-one mutations (position ctx-1 or ctx+1), which must
change the appended pool and the decode output.
"""
from __future__ import annotations

import numpy as np


def _slot(block_table_row: np.ndarray, block_size: int, pos: int) -> int:
    logical = pos // block_size
    return int(block_table_row[logical]) * block_size + pos % block_size


def decode_slot_mapping(block_tables: np.ndarray, context_lens: np.ndarray,
                        block_size: int) -> np.ndarray:
    """One new token per request at position context_lens[b] (pre-increment)."""
    bt = np.asarray(block_tables)
    ctx = np.asarray(context_lens)
    return np.array([_slot(bt[b], block_size, int(ctx[b])) for b in range(bt.shape[0])],
                    dtype=np.int64)


def prefill_slot_mapping(block_tables: np.ndarray, starts, counts, block_size: int,
                         pad_mask=None) -> np.ndarray:
    """Request r appends counts[r] tokens at positions starts[r] .. starts[r]+counts[r]-1;
    tokens are ordered request by request.  pad_mask (bool per token) marks
    padding tokens, whose slot is -1."""
    bt = np.asarray(block_tables)
    out = []
    for r, (s, c) in enumerate(zip(starts, counts)):
        for p in range(int(s), int(s) + int(c)):
            out.append(_slot(bt[r], block_size, p))
    out = np.array(out, dtype=np.int64)
    if pad_mask is not None:
        out[np.asarray(pad_mask, dtype=bool)] = -1
    return out


def slot_mapping_ref(token_request, token_position, block_tables, block_size: int,
                     batch: int) -> np.ndarray:
    """Slot id of every new token, from its request and position (the launcher's step).

    [Append] Inputs items 6 and 7 and step 9: with a block table, token t of request r at
    position p goes to block_tables[r, p // block_size] * block_size + p % block_size.
    Without one (block_tables None), the contiguous cache [batch, num_kv_heads, max_seq_len,
    head_dim] is meant and the id is r * max_seq_len + p with block_size = max_seq_len (the
    encoding of [Append] step 5; a reading, as Inputs item 6 states another).
    Readings: a token whose request is negative (padding), at or beyond `batch`, or whose
    position is negative or outside its table row (or >= max_seq_len) gets -1, so the append
    skips it.  token_request None means token t belongs to request t (one decode token each).
    """
    pos = np.asarray(token_position, dtype=np.int64)
    req = np.arange(pos.shape[0]) if token_request is None else np.asarray(token_request, np.int64)
    out = np.full(pos.shape[0], -1, dtype=np.int64)
    for t in range(pos.shape[0]):
        r, p = int(req[t]), int(pos[t])
        if r < 0 or r >= batch or p < 0:
            continue
        if block_tables is None:
            if p < block_size:
                out[t] = r * block_size + p
            continue
        row = np.asarray(block_tables)[r]
        if p // block_size < row.shape[0]:
            out[t] = _slot(row, block_size, p)
    return out

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

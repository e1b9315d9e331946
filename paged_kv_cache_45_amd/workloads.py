"""Seeded synthetic workloads for the paged KV-cache path.

This module only *generates* inputs: context lengths, a shuffled physical
block allocation, block tables, the slot ids of new tokens, and N(0,1)
tensors.  It holds none of the method's arithmetic (no quantisation, no
attention, no packing) and imports nothing from the oracle or from the HIP
binding, so that both sides of a parity check consume identical bytes.

Slot ids of new tokens come from the allocator's own bookkeeping: every
request owns a list of physical blocks, and the i-th token position of the
request lives at the i-th slot of that list.  (The oracle re-derives the same
slots from the block table and the context length; the tests compare the two.)

Shapes follow the pages' workloads:
  * "Triton KV Cache and PagedAttention" (llm-algo-leetcode ch. 10), Step 4
    test: batch 2, 4 heads, head_dim 64, block_size 16, 20 physical blocks,
    fp16 N(0,1), context lengths 10 and 25, and a literal two-row block table.
  * "Write Triton Kv Cache Append Kernel", Inputs and Performance requirements:
    new K/V of shape [num_tokens, num_kv_heads, head_dim], decode = one token
    per request, prefill = whole prompts, padding tokens marked with slot -1.
  * "triton-3bit-kv-cache-kernel" README, section 2: N(0,1) K/V tiles that are
    affine-quantised to uint3 with fp16 scale/zero per (token, kv head).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

# Bit patterns used to poison memory that a correct kernel never reads.
NAN_BITS = {torch.bfloat16: 0x7FC0, torch.float16: 0x7E00}

BASE_SEED = 42  # the seed of the pages' tiny PagedAttention test


@dataclasses.dataclass
class PagedWorkload:
    """One synthetic decode (and/or append) batch over a paged block pool."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: torch.dtype                 # q / new K,V / same-dtype cache element type
    ctx_before: torch.Tensor           # int32 [B] tokens already cached (pre-append)
    ctx_after: torch.Tensor            # int32 [B] attention length after the append
    block_tables: torch.Tensor         # int32 [B, max_blocks] (padding entries = 0)
    q: torch.Tensor                    # [B, Hq, D]
    k_pool: Optional[torch.Tensor]     # [NB, BS, Hkv, D] existing tokens (None for quantised pools)
    v_pool: Optional[torch.Tensor]
    new_k: Optional[torch.Tensor]      # [T, Hkv, D]
    new_v: Optional[torch.Tensor]
    slot_mapping: Optional[torch.Tensor]  # int64 [T]
    token_request: Optional[torch.Tensor]  # int64 [T] request of each new token (-1 = padding)
    token_position: Optional[torch.Tensor]  # int64 [T] position of each new token in its request
    blocks_of: List[List[int]]         # physical blocks owned by each request, in logical order
    sm_scale: float

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_context_len(self) -> int:
        return int(self.ctx_after.max().item()) if self.batch else 0


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _allocate(lens_needed: List[int], block_size: int, spare_frac: float, gen: torch.Generator,
              min_blocks: int = 0):
    """Give each request cdiv(len, BS) distinct physical blocks out of a shuffled pool."""
    need = [_cdiv(n, block_size) for n in lens_needed]
    total = sum(need)
    nb = max(total + int(math.ceil(spare_frac * total)), min_blocks)
    perm = torch.randperm(nb, generator=gen).tolist()
    blocks_of, off = [], 0
    for n in need:
        blocks_of.append(perm[off:off + n])
        off += n
    max_blocks = max(need) if need else 1
    bt = torch.zeros((len(need), max(max_blocks, 1)), dtype=torch.int32)
    for b, blks in enumerate(blocks_of):
        if blks:
            bt[b, :len(blks)] = torch.tensor(blks, dtype=torch.int32)
    return nb, blocks_of, bt


def _slot_of(blocks: List[int], block_size: int, pos: int) -> int:
    # allocator bookkeeping: the request's slots, enumerated in logical order
    return blocks[pos // block_size] * block_size + pos % block_size


def _randn(shape, dtype, device, gen):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def _device_gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def poison_unused(pool: torch.Tensor, blocks_of: List[List[int]], valid_len: List[int],
                  block_size: int) -> None:
    """Fill every slot that holds no live token of any request with NaN bits."""
    if pool.dtype not in NAN_BITS:
        raise TypeError("poisoning is defined for fp16/bf16 pools")
    nb = pool.shape[0]
    live = torch.zeros((nb, block_size), dtype=torch.bool)
    for blks, n in zip(blocks_of, valid_len):
        for i, blk in enumerate(blks):
            k = min(block_size, max(0, n - i * block_size))
            live[blk, :k] = True
    dead = (~live).to(pool.device)
    bits = pool.view(torch.int16)
    bits[dead] = NAN_BITS[pool.dtype] - (0x10000 if NAN_BITS[pool.dtype] >= 0x8000 else 0)


def decode_workload(name: str, *, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    block_size: int, ctx_lo: int, ctx_hi: int, dtype: torch.dtype, device,
                    seed: int, append_one: bool = True, spare_frac: float = 0.05,
                    poison: bool = True, ctx_override: Optional[List[int]] = None,
                    min_blocks: int = 0, make_pool: bool = True,
                    data_seed: Optional[int] = None) -> PagedWorkload:
    """A decode batch: ctx ~ U{ctx_lo..ctx_hi} tokens already cached per request,
    optionally one new token per request appended at position ctx, then one query
    token per request attending over the result.  `seed` draws the structure (lengths,
    block allocation); `data_seed` (default: seed) draws the tensors."""
    gen = torch.Generator().manual_seed(seed)
    if ctx_override is not None:
        ctx = list(ctx_override)
    else:
        ctx = torch.randint(ctx_lo, ctx_hi + 1, (batch,), generator=gen).tolist()
    after = [c + 1 for c in ctx] if append_one else list(ctx)
    nb, blocks_of, bt = _allocate(after, block_size, spare_frac, gen, min_blocks)
    dgen = _device_gen(device, seed if data_seed is None else data_seed)
    q = _randn((batch, num_q_heads, head_dim), dtype, device, dgen)
    k_pool = v_pool = None
    if make_pool:
        k_pool = _randn((nb, block_size, num_kv_heads, head_dim), dtype, device, dgen)
        v_pool = _randn((nb, block_size, num_kv_heads, head_dim), dtype, device, dgen)
        if poison:
            # the appended slot is poisoned too: only the append may make it live
            poison_unused(k_pool, blocks_of, ctx, block_size)
            poison_unused(v_pool, blocks_of, ctx, block_size)
    new_k = new_v = slots = treq = tpos = None
    if append_one:
        new_k = _randn((batch, num_kv_heads, head_dim), dtype, device, dgen)
        new_v = _randn((batch, num_kv_heads, head_dim), dtype, device, dgen)
        slots = torch.tensor([_slot_of(blocks_of[b], block_size, ctx[b]) for b in range(batch)],
                             dtype=torch.int64)
        treq = torch.arange(batch, dtype=torch.int64)
        tpos = torch.tensor(ctx, dtype=torch.int64)
    return PagedWorkload(
        name=name, batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, num_blocks=nb, dtype=dtype,
        ctx_before=torch.tensor(ctx, dtype=torch.int32),
        ctx_after=torch.tensor(after, dtype=torch.int32),
        block_tables=bt, q=q, k_pool=k_pool, v_pool=v_pool, new_k=new_k, new_v=new_v,
        slot_mapping=slots, token_request=treq, token_position=tpos, blocks_of=blocks_of,
        sm_scale=1.0 / math.sqrt(head_dim))


def literal_tiny_case(device) -> PagedWorkload:
    """The pages' own tiny PagedAttention check: 20 blocks of 16 slots, 4 heads of 64,
    context lengths 10 and 25, block table rows [5,0,0,0,0] and [12,3,0,0,0]; no append.
    ("Triton KV Cache and PagedAttention", Step 4 test.)  Data are N(0,1) fp16 from our
    own seeded generator (the page draws them with torch's global RNG on its GPU)."""
    B, H, D, BS, NB = 2, 4, 64, 16, 20
    dgen = _device_gen(device, BASE_SEED)
    q = _randn((B, H, D), torch.float16, device, dgen)
    k_pool = _randn((NB, BS, H, D), torch.float16, device, dgen)
    v_pool = _randn((NB, BS, H, D), torch.float16, device, dgen)
    bt = torch.tensor([[5, 0, 0, 0, 0], [12, 3, 0, 0, 0]], dtype=torch.int32)
    ctx = torch.tensor([10, 25], dtype=torch.int32)
    return PagedWorkload(
        name="literal-tiny", batch=B, num_q_heads=H, num_kv_heads=H, head_dim=D, block_size=BS,
        num_blocks=NB, dtype=torch.float16, ctx_before=ctx, ctx_after=ctx.clone(), block_tables=bt,
        q=q, k_pool=k_pool, v_pool=v_pool, new_k=None, new_v=None, slot_mapping=None,
        token_request=None, token_position=None, blocks_of=[[5], [12, 3]], sm_scale=1.0 / 8.0)


def tiny(device, seed: int = BASE_SEED + 1, poison: bool = True) -> PagedWorkload:
    """Tiny paged decode + append: B=2, Hq=Hkv=4, D=64, BS=16, 20 blocks, fp16,
    context lengths [10, 25] before appending one decode token per request."""
    return decode_workload("tiny", batch=2, num_q_heads=4, num_kv_heads=4, head_dim=64,
                           block_size=16, ctx_lo=0, ctx_hi=0, dtype=torch.float16, device=device,
                           seed=seed, ctx_override=[10, 25], min_blocks=20, spare_frac=0.0,
                           poison=poison)


def llama8b_decode(device, seed: int = BASE_SEED + 2, poison: bool = True,
                   batch: int = 64, make_pool: bool = True,
                   data_seed: Optional[int] = None) -> PagedWorkload:
    """Llama-8B-shaped decode step: B=64, 32 q heads / 8 kv heads, D=128, BS=16,
    bf16, ctx ~ U{512..4096}, one token appended per request, shuffled pool with
    5% spare (poisoned) blocks."""
    return decode_workload("llama8b-decode", batch=batch, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=16, ctx_lo=512, ctx_hi=4096,
                           dtype=torch.bfloat16, device=device, seed=seed, poison=poison,
                           make_pool=make_pool, data_seed=data_seed)


def long_context(device, seed: int = BASE_SEED + 4, poison: bool = False,
                 batch: int = 8, ctx_lo: int = 32768, ctx_hi: int = 131072) -> PagedWorkload:
    """Long-context split-K decode: B=8, 64 q heads / 8 kv heads, D=128, BS=64,
    bf16, ctx ~ U{32k..128k}, shuffled pool, no append."""
    return decode_workload("long-context", batch=batch, num_q_heads=64, num_kv_heads=8,
                           head_dim=128, block_size=64, ctx_lo=ctx_lo, ctx_hi=ctx_hi,
                           dtype=torch.bfloat16, device=device, seed=seed, append_one=False,
                           poison=poison)


@dataclasses.dataclass
class AppendWorkload:
    """A mixed prefill + decode append batch (no query)."""

    name: str
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: torch.dtype
    new_k: torch.Tensor           # [T, Hkv, D] (possibly a strided view)
    new_v: torch.Tensor
    slot_mapping: torch.Tensor    # int64 [T], -1 = padding
    token_request: torch.Tensor   # int64 [T]
    token_position: torch.Tensor  # int64 [T]
    block_tables: torch.Tensor    # int32 [R, max_blocks]
    blocks_of: List[List[int]]
    req_start: List[int]          # first position each request appends at
    req_count: List[int]          # tokens each request appends


def mixed_append(device, seed: int = BASE_SEED + 3, *, num_prompts: int = 8, prompt_lo: int = 128,
                 prompt_hi: int = 2048, num_decode: int = 56, ctx_lo: int = 128,
                 ctx_hi: int = 2048, num_kv_heads: int = 8, head_dim: int = 128,
                 block_size: int = 32, pad_frac: float = 0.10, dtype=torch.bfloat16,
                 qkv_view: bool = False, num_q_heads: int = 32) -> AppendWorkload:
    """Mixed prefill + decode append: num_prompts whole prompts from position 0
    (lengths U{prompt_lo..prompt_hi}), then one decode token for each of num_decode
    other requests at position ctx ~ U{ctx_lo..ctx_hi}; token order is prompts then
    decodes; round(pad_frac*T) seeded random entries of slot_mapping are set to -1.

    With qkv_view=True the new K/V are non-contiguous views into one fused
    [T, (Hq + 2*Hkv)*D] projection output, as the append page warns they often are."""
    gen = torch.Generator().manual_seed(seed)
    plens = torch.randint(prompt_lo, prompt_hi + 1, (num_prompts,), generator=gen).tolist()
    dctx = torch.randint(ctx_lo, ctx_hi + 1, (num_decode,), generator=gen).tolist()
    starts = [0] * num_prompts + dctx
    counts = plens + [1] * num_decode
    lens_after = [s + c for s, c in zip(starts, counts)]
    nb, blocks_of, bt = _allocate(lens_after, block_size, 0.0, gen)
    treq, tpos, slots = [], [], []
    for r, (s, c) in enumerate(zip(starts, counts)):
        for p in range(s, s + c):
            treq.append(r)
            tpos.append(p)
            slots.append(_slot_of(blocks_of[r], block_size, p))
    T = len(slots)
    npad = int(round(pad_frac * T))
    pad_idx = torch.randperm(T, generator=gen)[:npad]
    slots_t = torch.tensor(slots, dtype=torch.int64)
    treq_t = torch.tensor(treq, dtype=torch.int64)
    slots_t[pad_idx] = -1
    treq_t[pad_idx] = -1
    dgen = _device_gen(device, seed)
    if qkv_view:
        width = (num_q_heads + 2 * num_kv_heads) * head_dim
        qkv = _randn((T, width), dtype, device, dgen)
        k0 = num_q_heads * head_dim
        v0 = k0 + num_kv_heads * head_dim
        new_k = qkv[:, k0:v0].view(T, num_kv_heads, head_dim)
        new_v = qkv[:, v0:].view(T, num_kv_heads, head_dim)
    else:
        new_k = _randn((T, num_kv_heads, head_dim), dtype, device, dgen)
        new_v = _randn((T, num_kv_heads, head_dim), dtype, device, dgen)
    return AppendWorkload(
        name="mixed-append", num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=nb, dtype=dtype, new_k=new_k, new_v=new_v, slot_mapping=slots_t,
        token_request=treq_t, token_position=torch.tensor(tpos, dtype=torch.int64),
        block_tables=bt, blocks_of=blocks_of, req_start=starts, req_count=counts)


def packed3_decode(device, seed: int = BASE_SEED + 5, batch: int = 32,
                   ctx_lo: int = 1024, ctx_hi: int = 16384):
    """3-bit packed KV decode: B=32, 32 q / 8 kv heads, D=128, BS=16,
    ctx ~ U{1k..16k}.  Returns the decode structure plus the raw fp16 N(0,1)
    K/V of every live token (token order = request-major) and its slot ids; the
    u3 pool is produced by appending them through the 3-bit quantiser."""
    wl = decode_workload("packed3-decode", batch=batch, num_q_heads=32, num_kv_heads=8,
                         head_dim=128, block_size=16, ctx_lo=ctx_lo, ctx_hi=ctx_hi,
                         dtype=torch.float16, device=device, seed=seed, append_one=False,
                         poison=False, make_pool=False)
    slots = []
    for b in range(batch):
        L = int(wl.ctx_after[b])
        slots.extend(_slot_of(wl.blocks_of[b], wl.block_size, p) for p in range(L))
    T = len(slots)
    dgen = _device_gen(device, seed + 1000)
    k_all = _randn((T, wl.num_kv_heads, wl.head_dim), torch.float16, device, dgen)
    v_all = _randn((T, wl.num_kv_heads, wl.head_dim), torch.float16, device, dgen)
    wl.new_k, wl.new_v = k_all, v_all
    wl.slot_mapping = torch.tensor(slots, dtype=torch.int64)
    return wl


def random_u3_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                   device, seed: int):
    """Uniformly random packed words and random positive fp16 (scale, zero) pairs:
    a u3 pool that is valid by construction, for decode tests independent of the
    quantiser.  Returns (words int32 [NB,BS,Hkv,D*3/32], meta fp16 [NB,BS,Hkv,2])."""
    g = torch.Generator().manual_seed(seed)
    words = torch.randint(-2**31, 2**31, (num_blocks, block_size, num_kv_heads, head_dim * 3 // 32),
                          generator=g, dtype=torch.int64).to(torch.int32)
    s = torch.rand((num_blocks, block_size, num_kv_heads), generator=g) * 0.9 + 0.1
    z = torch.rand((num_blocks, block_size, num_kv_heads), generator=g) * 7.0
    meta = torch.stack([s, z], dim=-1).to(torch.float16)
    return words.to(device), meta.to(device)

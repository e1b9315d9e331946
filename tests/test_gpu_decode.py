"""GPU parity of paged_decode against the float64 oracle (max abs error <= 2e-3).

"Triton KV Cache and PagedAttention": Step 1 and the reference answer (block-table
indirection, masking past the context, online softmax), the Step 4 test (tiny case,
tolerance 2e-3).  GQA per "Write Triton Kv Cache Append Kernel" (Kernel design rules).
3-bit cache per "triton-3bit-kv-cache-kernel" README (title paragraph, section 2).
Split-K partitions merged by log-sum-exp.
"""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import need_gpu, bits16, np_u32, dtype_name, f32_of, report, ATTN_TOL
from paged_kv_cache_45_amd import workloads as W
import oracle
from oracle import PoolView, paged_decode_ref, quantize_u3_rows, pack_rows_u3, quantize_fp8_rows

pytestmark = pytest.mark.gpu


def _oracle_same(wl, k_pool, v_pool, ctx, heads=None):
    dn = dtype_name(wl.dtype)
    return paged_decode_ref(f32_of(wl.q), PoolView("same", bits16(k_pool), dtype=dn),
                            PoolView("same", bits16(v_pool), dtype=dn), wl.block_tables.numpy(),
                            ctx.numpy(), wl.block_size, wl.num_kv_heads, wl.sm_scale, heads=heads)


def _decode(P, wl, k_pool, v_pool, ctx, **kw):
    return P.paged_decode(wl.q, k_pool, v_pool, wl.block_tables.cuda(), ctx.cuda(),
                          int(ctx.max()), wl.sm_scale, **kw)


def test_tiny_append_then_decode():
    P = need_gpu()
    wl = W.tiny("cuda")
    kc, vc = wl.k_pool.clone(), wl.v_pool.clone()
    P.kv_append(wl.new_k, wl.new_v, wl.slot_mapping.cuda(), kc, vc)
    out = _decode(P, wl, kc, vc, wl.ctx_after)
    # the oracle appends on its own copy of the pool
    hk, hv = bits16(wl.k_pool).copy(), bits16(wl.v_pool).copy()
    oracle.append_ref(bits16(wl.new_k), bits16(wl.new_v), wl.slot_mapping.numpy(), hk, hv,
                      oracle.CacheSpec("same", "f16"), wl.block_size)
    want = paged_decode_ref(f32_of(wl.q), PoolView("same", hk, dtype="f16"),
                            PoolView("same", hv, dtype="f16"), wl.block_tables.numpy(),
                            wl.ctx_after.numpy(), wl.block_size, wl.num_kv_heads, wl.sm_scale)
    assert report("tiny", f32_of(out), want, wl.dtype) <= ATTN_TOL


def test_literal_tiny_case():
    P = need_gpu()
    wl = W.literal_tiny_case("cuda")
    out = _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_after)
    want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_after)
    assert report("literal", f32_of(out), want, wl.dtype) <= ATTN_TOL


def test_llama8b_full_size_all_heads():
    """Llama-8B-shaped step at full size: append one token per request, decode, compare all
    64 x 32 outputs (poisoned spare blocks and tail slots)."""
    P = need_gpu()
    wl = W.llama8b_decode("cuda")
    kc, vc = wl.k_pool.clone(), wl.v_pool.clone()
    P.kv_append(wl.new_k, wl.new_v, wl.slot_mapping.cuda(), kc, vc)
    out = _decode(P, wl, kc, vc, wl.ctx_after)
    hk, hv = bits16(wl.k_pool).copy(), bits16(wl.v_pool).copy()
    oracle.append_ref(bits16(wl.new_k), bits16(wl.new_v), wl.slot_mapping.numpy(), hk, hv,
                      oracle.CacheSpec("same", "bf16"), wl.block_size)
    assert np.array_equal(bits16(kc), hk) and np.array_equal(bits16(vc), hv)
    want = paged_decode_ref(f32_of(wl.q), PoolView("same", hk, dtype="bf16"),
                            PoolView("same", hv, dtype="bf16"), wl.block_tables.numpy(),
                            wl.ctx_after.numpy(), wl.block_size, wl.num_kv_heads, wl.sm_scale)
    assert report("llama8b", f32_of(out), want, wl.dtype) <= ATTN_TOL


@pytest.mark.parametrize("Hq,Hkv,D,bs", [(32, 8, 128, 16), (64, 8, 128, 16), (16, 8, 64, 16),
                                         (8, 8, 128, 32)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_many_requests_few_partials(Hq, Hkv, D, bs, dtype):
    """72 requests: enough that a split segment holds only a few partial states, which the merge
    takes in one pass, several elements per thread.  Empty, one-token and ragged contexts, all
    heads, NaN-poisoned unused slots."""
    P = need_gpu()
    rng = np.random.default_rng(900 + Hq + D + bs)
    lens = rng.integers(2, 700, size=72)
    lens[[0, 5, 17, 40, 71]] = 0
    lens[[1, 33]] = 1
    wl = W.decode_workload("few-partials", batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv,
                           head_dim=D, block_size=bs, ctx_lo=0, ctx_hi=0, dtype=dtype, device="cuda",
                           seed=W.BASE_SEED + 51, append_one=False, ctx_override=[int(x) for x in lens])
    out = _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_after)
    want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_after)
    assert np.all(f32_of(out)[lens == 0] == 0)
    assert report(f"few partials Hq{Hq} D{D} bs{bs} {dtype_name(dtype)}", f32_of(out), want,
                  dtype) <= ATTN_TOL


@pytest.mark.parametrize("ps", [0, 16, 256, 512, 4096])
def test_partition_sizes_agree(ps):
    P = need_gpu()
    wl = W.llama8b_decode("cuda", batch=6)
    out = _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_before, partition_size=ps)
    want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_before)
    assert report(f"partition {ps}", f32_of(out), want, wl.dtype) <= ATTN_TOL


def test_long_context_split_k_sampled():
    """Long-context split-K at full size (B=8, 64/8 heads, BS 64, 32k-128k tokens,
    partitions of 512), oracle on two requests x all 64 heads."""
    P = need_gpu()
    wl = W.long_context("cuda")
    out = _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_after, partition_size=512)
    heads = [(b, h) for b in (0, 5) for h in range(wl.num_q_heads)]
    want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_after, heads=heads)
    got = f32_of(out)
    sel = np.array([b for b, _ in heads]), np.array([h for _, h in heads])
    assert report("long-context", got[sel], want[sel], wl.dtype) <= ATTN_TOL


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("D,bs", [(128, 16), (64, 16), (128, 32), (64, 64)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_shapes_ragged(G, D, bs, dtype):
    P = need_gpu()
    Hkv = 2
    lens = [1, 15, 16, 17, 511, 512, 513, 1000, 0, 33]
    wl = W.decode_workload("ragged", batch=len(lens), num_q_heads=G * Hkv, num_kv_heads=Hkv,
                           head_dim=D, block_size=bs, ctx_lo=0, ctx_hi=0, dtype=dtype,
                           device="cuda", seed=100 + G + D + bs, append_one=False,
                           ctx_override=lens)
    for ps in (0, 16, 512):
        out = _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_after, partition_size=ps)
        want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_after)
        got = f32_of(out)
        assert np.all(got[lens.index(0)] == 0)
        assert report(f"G{G} D{D} bs{bs} {dtype} ps{ps}", got, want, dtype) <= ATTN_TOL


def test_strided_q_and_out_views():
    P = need_gpu()
    wl = W.llama8b_decode("cuda", batch=3)
    big = torch.randn((3, 2 * wl.num_q_heads, 2 * wl.head_dim), device="cuda").to(wl.dtype)
    q = big[:, ::2, :wl.head_dim]
    q.copy_(wl.q)
    wl.q = q
    obuf = torch.zeros((3, wl.num_q_heads, 3 * wl.head_dim), device="cuda", dtype=wl.dtype)
    out = obuf[:, :, wl.head_dim:2 * wl.head_dim]
    _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_before, out=out)
    want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_before)
    assert report("strided", f32_of(out), want, wl.dtype) <= ATTN_TOL
    assert torch.all(obuf[:, :, :wl.head_dim] == 0) and torch.all(obuf[:, :, 2 * wl.head_dim:] == 0)


def _u3_pools_from_raw(wl, k_all, v_all, slots):
    """Oracle side: quantise the raw fp16 rows with the oracle and scatter them into pools."""
    NB, BS, H, D = wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim
    pools = []
    for raw in (k_all, v_all):
        x = raw.float().cpu().numpy()
        q, s16, z16 = quantize_u3_rows(x)
        words = np.zeros((NB * BS, H, D * 3 // 32), dtype=np.uint32)
        meta = np.zeros((NB * BS, H, 2), dtype=np.float16)
        sl = slots.numpy()
        words[sl] = pack_rows_u3(q)
        meta[sl, :, 0] = s16
        meta[sl, :, 1] = z16
        pools.append(PoolView("u3", words.reshape(NB, BS, H, -1), meta.reshape(NB, BS, H, 2),
                              head_dim=D))
    return pools


def _u3_case(P, batch, ctx_lo, ctx_hi, seed, sample=None, qdtype=torch.float16, workspace=None):
    wl = W.packed3_decode("cuda", seed=seed, batch=batch, ctx_lo=ctx_lo, ctx_hi=ctx_hi)
    NB, BS, H, D = wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim
    kc = torch.zeros((NB, BS, H, D * 3 // 32), dtype=torch.int32, device="cuda")
    vc = torch.zeros_like(kc)
    km = torch.zeros((NB, BS, H, 2), dtype=torch.float16, device="cuda")
    vm = torch.zeros_like(km)
    P.kv_append(wl.new_k, wl.new_v, wl.slot_mapping.cuda(), kc, vc, km, vm, cache_dtype="u3")
    q = wl.q.to(qdtype)
    out = P.paged_decode(q, kc, vc, wl.block_tables.cuda(), wl.ctx_after.cuda(),
                         int(wl.ctx_after.max()), wl.sm_scale, k_meta=km, v_meta=vm,
                         cache_dtype="u3", workspace=workspace)
    kpool, vpool = _u3_pools_from_raw(wl, wl.new_k, wl.new_v, wl.slot_mapping)
    assert np.array_equal(np_u32(kc), kpool.cache) and np.array_equal(np_u32(vc), vpool.cache)
    assert np.array_equal(km.cpu().numpy().view(np.uint16), kpool.meta.view(np.uint16))
    assert np.array_equal(vm.cpu().numpy().view(np.uint16), vpool.meta.view(np.uint16))
    want = paged_decode_ref(f32_of(q), kpool, vpool, wl.block_tables.numpy(), wl.ctx_after.numpy(),
                            BS, H, wl.sm_scale, heads=sample)
    got = f32_of(out)
    if sample is not None:
        sel = np.array([b for b, _ in sample]), np.array([h for _, h in sample])
        got, want = got[sel], want[sel]
    return got, want


def test_u3_decode_small():
    P = need_gpu()
    got, want = _u3_case(P, batch=4, ctx_lo=1, ctx_hi=700, seed=11)
    assert report("u3 small", got, want) <= ATTN_TOL


def test_u3_decode_bf16_query():
    P = need_gpu()
    got, want = _u3_case(P, batch=3, ctx_lo=100, ctx_hi=900, seed=12, qdtype=torch.bfloat16)
    assert report("u3 bf16 q", got, want, torch.bfloat16) <= ATTN_TOL


def test_u3_decode_full_size_sampled():
    """3-bit decode at full size (B=32, 32/8 heads, BS 16, 1k-16k), append through the u3
    quantiser, oracle on 3 requests x all heads."""
    P = need_gpu()
    sample = [(b, h) for b in (0, 13, 31) for h in range(32)]
    got, want = _u3_case(P, batch=32, ctx_lo=1024, ctx_hi=16384, seed=W.BASE_SEED + 5,
                         sample=sample)
    assert report("u3 full", got, want) <= ATTN_TOL


def test_random_u3_pool_decode():
    """Decode over a u3 pool of uniformly random words and (scale, zero) pairs."""
    P = need_gpu()
    wl = W.decode_workload("u3-random", batch=5, num_q_heads=16, num_kv_heads=4, head_dim=128,
                           block_size=32, ctx_lo=1, ctx_hi=1500, dtype=torch.float16, device="cuda",
                           seed=21, append_one=False, make_pool=False)
    words, meta = W.random_u3_pool(wl.num_blocks, 32, 4, 128, "cuda", seed=22)
    words2, meta2 = W.random_u3_pool(wl.num_blocks, 32, 4, 128, "cuda", seed=23)
    out = P.paged_decode(wl.q, words, words2, wl.block_tables.cuda(), wl.ctx_after.cuda(),
                         int(wl.ctx_after.max()), wl.sm_scale, k_meta=meta, v_meta=meta2,
                         cache_dtype="u3")
    kp = PoolView("u3", np_u32(words), meta.cpu().numpy(), head_dim=128)
    vp = PoolView("u3", np_u32(words2), meta2.cpu().numpy(), head_dim=128)
    want = paged_decode_ref(f32_of(wl.q), kp, vp, wl.block_tables.numpy(), wl.ctx_after.numpy(),
                            32, 4, wl.sm_scale)
    assert report("u3 random pool", f32_of(out), want) <= ATTN_TOL


def test_rejects_bad_arguments():
    P = need_gpu()
    wl = W.tiny("cuda")
    with pytest.raises(P.PagedKVError):      # group size 3
        P.paged_decode(torch.zeros((2, 6, 64), dtype=torch.float16, device="cuda"),
                       wl.k_pool[:, :, :2], wl.v_pool[:, :, :2], wl.block_tables.cuda(),
                       wl.ctx_after.cuda(), 26)
    with pytest.raises(P.PagedKVError):      # workspace too small
        P.paged_decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables.cuda(), wl.ctx_after.cuda(), 26,
                       partition_size=16, workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"))


def test_workspace_reused_across_calls():
    """One workspace serves consecutive calls of different batch sizes and partition sizes: each
    call overwrites every partial state and segment record it reads."""
    P = need_gpu()
    big = W.llama8b_decode("cuda", batch=48, seed=W.BASE_SEED + 21)
    small = W.llama8b_decode("cuda", batch=5, seed=W.BASE_SEED + 22)
    ws = P.decode_workspace(big.batch, big.num_q_heads, big.num_kv_heads, big.head_dim,
                            int(big.ctx_before.max()), 16)
    for rep, (wl, ps) in enumerate([(big, 0), (small, 0), (big, 16), (small, 64), (big, 0)]):
        need = P.paged_decode_workspace_size(wl.batch, wl.num_q_heads, wl.num_kv_heads,
                                             wl.head_dim, int(wl.ctx_before.max()), ps)
        assert need <= ws.numel()
        out = _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_before, partition_size=ps, workspace=ws)
        heads = [(b, h) for b in range(min(wl.batch, 6)) for h in range(wl.num_q_heads)]
        want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_before, heads=heads)
        sel = np.array([b for b, _ in heads]), np.array([h for _, h in heads])
        assert report(f"reuse {rep} B={wl.batch} ps={ps}", f32_of(out)[sel], want[sel],
                      wl.dtype) <= ATTN_TOL


def test_large_blocks_ragged():
    """64-token blocks (128 KB of a wave's K/V per block), contexts shared by several
    workgroups: ragged lengths, one-block and one-token contexts, all heads; the same workspace
    three times."""
    P = need_gpu()
    lens = [1, 63, 64, 65, 5000, 20011, 129, 12345]
    wl = W.decode_workload("large-blocks", batch=len(lens), num_q_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=64, ctx_lo=0, ctx_hi=0, dtype=torch.bfloat16, device="cuda",
                           seed=W.BASE_SEED + 31, append_one=False, ctx_override=lens)
    ws = P.decode_workspace(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, max(lens), 0)
    want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_after)
    for rep in range(3):
        out = _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_after, workspace=ws)
        assert report(f"large blocks rep {rep}", f32_of(out), want, wl.dtype) <= ATTN_TOL


@pytest.mark.parametrize("fill", ["small-counts", "ones", "random"])
def test_workspace_any_contents(fill):
    """The workspace may hold anything when a call starts: filled before each of three calls with
    small counts, all-ones bytes or random bytes, the decode over 64-token blocks and long
    contexts matches the oracle at partition sizes 16 and 512."""
    P = need_gpu()
    lens = [1, 63, 64, 65, 5000, 20011, 129, 12345]
    wl = W.decode_workload("dirty-workspace", batch=len(lens), num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=64, ctx_lo=0, ctx_hi=0, dtype=torch.bfloat16,
                           device="cuda", seed=W.BASE_SEED + 32, append_one=False, ctx_override=lens)
    want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_after)
    for ps in (0, 512):
        n = P.paged_decode_workspace_size(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                          max(lens), ps)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        gen = torch.Generator(device="cuda").manual_seed(7)
        for rep in range(3):
            if fill == "small-counts":
                ws.view(torch.int32)[: n // 4 // 2].fill_(rep + 1)
            elif fill == "ones":
                ws.fill_(0xFF)
            else:
                ws.copy_(torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=gen))
            out = _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_after, partition_size=ps, workspace=ws)
            assert report(f"dirty workspace {fill} ps={ps} rep {rep}", f32_of(out), want,
                          wl.dtype) <= ATTN_TOL


# ---- fp8 e4m3fn cache (one fp32 scale per (slot, kv head)) ---------------------------------
# The GPU pools come from kv_append's fp8 quantiser over every slot of a bf16/fp16 pool; the
# oracle quantises the same rows itself, the live rows of both must agree bit for bit, and the
# oracle's decode reads only its own pools.

def _live_slots(wl, lens, blocks=None):
    """bool [NB, BS]: slots holding a live token of some request (of `blocks` only, if given)."""
    live = np.zeros((wl.num_blocks, wl.block_size), dtype=bool)
    for blks, n in zip(wl.blocks_of, lens):
        for i, blk in enumerate(blks):
            if blocks is None or blk in blocks:
                live[blk, :min(wl.block_size, max(0, int(n) - i * wl.block_size))] = True
    return live


def _fp8_pools_gpu(P, wl):
    NB, BS, H, D = wl.k_pool.shape
    kc = torch.empty((NB, BS, H, D), dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    km = torch.empty((NB, BS, H), dtype=torch.float32, device="cuda")
    vm = torch.empty_like(km)
    slots = torch.arange(NB * BS, dtype=torch.int64, device="cuda")
    P.kv_append(wl.k_pool.reshape(NB * BS, H, D), wl.v_pool.reshape(NB * BS, H, D), slots,
                kc, vc, km, vm)
    return kc, vc, km, vm


def _fp8_pools_oracle(wl, live):
    """Oracle codes and scales of the live rows (zeros / ones elsewhere)."""
    NB, BS, H, D = wl.k_pool.shape
    pools = []
    for pool in (wl.k_pool, wl.v_pool):
        codes = np.zeros((NB, BS, H, D), dtype=np.uint8)
        scales = np.ones((NB, BS, H), dtype=np.float32)
        c, s = quantize_fp8_rows(f32_of(pool)[live])
        codes[live], scales[live] = c, s
        pools.append(PoolView("fp8", codes, scales))
    return pools


def _fp8_check_pools(gpu, kpool, vpool, live):
    kc, vc, km, vm = gpu
    assert np.array_equal(kc.cpu().numpy()[live], kpool.cache[live])
    assert np.array_equal(vc.cpu().numpy()[live], vpool.cache[live])
    assert np.array_equal(km.cpu().numpy()[live].view(np.uint32), kpool.meta[live].view(np.uint32))
    assert np.array_equal(vm.cpu().numpy()[live].view(np.uint32), vpool.meta[live].view(np.uint32))


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("D,bs", [(128, 16), (64, 64), (128, 32)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_fp8_decode_shapes_ragged(G, D, bs, dtype):
    P = need_gpu()
    Hkv = 2
    lens = [1, 15, 16, 17, 511, 512, 513, 1000, 0, 33]
    wl = W.decode_workload("fp8-ragged", batch=len(lens), num_q_heads=G * Hkv, num_kv_heads=Hkv,
                           head_dim=D, block_size=bs, ctx_lo=0, ctx_hi=0, dtype=dtype,
                           device="cuda", seed=200 + G + D + bs, append_one=False,
                           ctx_override=lens)
    gpu = _fp8_pools_gpu(P, wl)
    live = _live_slots(wl, lens)
    kpool, vpool = _fp8_pools_oracle(wl, live)
    _fp8_check_pools(gpu, kpool, vpool, live)
    want = paged_decode_ref(f32_of(wl.q), kpool, vpool, wl.block_tables.numpy(), np.array(lens),
                            bs, Hkv, wl.sm_scale)
    for ps in (0, 512):
        out = P.paged_decode(wl.q, gpu[0], gpu[1], wl.block_tables.cuda(), wl.ctx_after.cuda(),
                             max(lens), wl.sm_scale, k_meta=gpu[2], v_meta=gpu[3], partition_size=ps)
        got = f32_of(out)
        assert np.all(got[lens.index(0)] == 0)
        assert report(f"fp8 G{G} D{D} bs{bs} {dtype} ps{ps}", got, want, dtype) <= ATTN_TOL


def test_fp8_decode_llama8b_full_size_sampled():
    """The Llama-8B step's shape (B=64, 32/8 heads, D=128, BS 16, bf16 q, U{512..4096}) over
    fp8 pools, at the launch configuration the fp8 bench line times; oracle on 3 requests."""
    P = need_gpu()
    wl = W.llama8b_decode("cuda")
    gpu = _fp8_pools_gpu(P, wl)
    ctx = wl.ctx_before.numpy()
    sample_b = (0, 29, 63)
    blocks = {blk for b in sample_b for blk in wl.blocks_of[b]}
    live = _live_slots(wl, ctx, blocks)
    kpool, vpool = _fp8_pools_oracle(wl, live)
    _fp8_check_pools(gpu, kpool, vpool, live)
    out = P.paged_decode(wl.q, gpu[0], gpu[1], wl.block_tables.cuda(), wl.ctx_before.cuda(),
                         int(ctx.max()), wl.sm_scale, k_meta=gpu[2], v_meta=gpu[3])
    heads = [(b, h) for b in sample_b for h in range(wl.num_q_heads)]
    want = paged_decode_ref(f32_of(wl.q), kpool, vpool, wl.block_tables.numpy(), ctx,
                            wl.block_size, wl.num_kv_heads, wl.sm_scale, heads=heads)
    sel = np.array([b for b, _ in heads]), np.array([h for _, h in heads])
    assert report("fp8 llama8b", f32_of(out)[sel], want[sel], wl.dtype) <= ATTN_TOL


def test_fp8_decode_large_blocks_ragged():
    """fp8 pools with 64-token blocks (a wave's share of a block is 66 KB of codes and scales),
    ragged contexts shared by several workgroups; the same workspace three times."""
    P = need_gpu()
    lens = [1, 63, 64, 65, 5000, 20011, 129, 12345]
    wl = W.decode_workload("fp8-large-blocks", batch=len(lens), num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=64, ctx_lo=0, ctx_hi=0, dtype=torch.bfloat16,
                           device="cuda", seed=W.BASE_SEED + 32, append_one=False, ctx_override=lens)
    gpu = _fp8_pools_gpu(P, wl)
    live = _live_slots(wl, lens)
    kpool, vpool = _fp8_pools_oracle(wl, live)
    _fp8_check_pools(gpu, kpool, vpool, live)
    want = paged_decode_ref(f32_of(wl.q), kpool, vpool, wl.block_tables.numpy(), np.array(lens),
                            wl.block_size, wl.num_kv_heads, wl.sm_scale)
    ws = P.decode_workspace(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, max(lens), 0)
    for rep in range(3):
        out = P.paged_decode(wl.q, gpu[0], gpu[1], wl.block_tables.cuda(), wl.ctx_after.cuda(),
                             max(lens), wl.sm_scale, k_meta=gpu[2], v_meta=gpu[3], workspace=ws)
        assert report(f"fp8 large blocks rep {rep}", f32_of(out), want, wl.dtype) <= ATTN_TOL


def test_one_workspace_serves_every_cache_kind():
    """A workspace sized by paged_decode_workspace_size (which plans for every cache kind) serves
    bf16, fp8 and 3-bit decodes over 64-token blocks in turn, each on what the one before left."""
    P = need_gpu()
    lens = [700, 1, 4100, 64, 0, 2048]
    same = W.decode_workload("mix-same", batch=len(lens), num_q_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=64, ctx_lo=0, ctx_hi=0, dtype=torch.bfloat16, device="cuda",
                             seed=W.BASE_SEED + 41, append_one=False, ctx_override=lens)
    gpu = _fp8_pools_gpu(P, same)
    live = _live_slots(same, lens)
    kpool8, vpool8 = _fp8_pools_oracle(same, live)
    want_same = _oracle_same(same, same.k_pool, same.v_pool, same.ctx_after)
    want_fp8 = paged_decode_ref(f32_of(same.q), kpool8, vpool8, same.block_tables.numpy(), np.array(lens),
                                same.block_size, same.num_kv_heads, same.sm_scale)
    ws = P.decode_workspace(same.batch, same.num_q_heads, same.num_kv_heads, same.head_dim, max(lens), 0)
    for rep in range(2):
        out = _decode(P, same, same.k_pool, same.v_pool, same.ctx_after, workspace=ws)
        assert report(f"mixed kinds bf16 {rep}", f32_of(out), want_same, same.dtype) <= ATTN_TOL
        out = P.paged_decode(same.q, gpu[0], gpu[1], same.block_tables.cuda(), same.ctx_after.cuda(),
                             max(lens), same.sm_scale, k_meta=gpu[2], v_meta=gpu[3], workspace=ws)
        assert report(f"mixed kinds fp8 {rep}", f32_of(out), want_fp8, same.dtype) <= ATTN_TOL
        got, want = _u3_case(P, batch=3, ctx_lo=100, ctx_hi=900, seed=13 + rep, workspace=ws)
        assert report(f"mixed kinds u3 {rep}", got, want) <= ATTN_TOL


@pytest.mark.parametrize("kind", ["same", "fp8"])
def test_dual_stacked_block_layout(kind):
    """The dual-stacked block layout [num_blocks, 2, num_kv_heads, block_size, head_dim] (K and V
    of a block in one buffer, head-major inside the block; "Write Triton Kv Cache Append Kernel",
    Inputs (cache layout) and Common failure modes) through the stride arguments: K and V are the
    two views buf[:, 0] and buf[:, 1] permuted to [block, slot, head, d]; append then decode,
    against the oracle on the same rows."""
    P = need_gpu()
    lens = [300, 17, 1025, 0, 64]
    wl = W.decode_workload("dual-stacked", batch=len(lens), num_q_heads=16, num_kv_heads=4, head_dim=128,
                           block_size=16, ctx_lo=0, ctx_hi=0, dtype=torch.bfloat16, device="cuda",
                           seed=W.BASE_SEED + 51, append_one=True, ctx_override=lens, poison=False)
    NB, BS, H, D = wl.k_pool.shape
    if kind == "same":
        buf = torch.empty((NB, 2, H, BS, D), dtype=wl.dtype, device="cuda")
        kc, vc = buf[:, 0].permute(0, 2, 1, 3), buf[:, 1].permute(0, 2, 1, 3)
        kc.copy_(wl.k_pool)
        vc.copy_(wl.v_pool)
        km = vm = None
    else:
        gpu = _fp8_pools_gpu(P, wl)
        buf = torch.empty((NB, 2, H, BS, D), dtype=torch.uint8, device="cuda")
        kc, vc = buf[:, 0].permute(0, 2, 1, 3), buf[:, 1].permute(0, 2, 1, 3)
        kc.copy_(gpu[0])
        vc.copy_(gpu[1])
        km, vm = gpu[2], gpu[3]
    assert kc.stride() == (2 * H * BS * D, D, BS * D, 1)
    # the new token of every request through the strided pools
    if kind == "same":
        P.kv_append(wl.new_k, wl.new_v, wl.slot_mapping.cuda(), kc, vc)
        dn = dtype_name(wl.dtype)
        kpool = PoolView("same", bits16(kc), dtype=dn)
        vpool = PoolView("same", bits16(vc), dtype=dn)
        kref, vref = bits16(wl.k_pool).copy(), bits16(wl.v_pool).copy()
        oracle.append_ref(bits16(wl.new_k), bits16(wl.new_v), wl.slot_mapping.numpy(), kref, vref,
                          oracle.CacheSpec("same", dn), BS)
        assert np.array_equal(kpool.cache, kref) and np.array_equal(vpool.cache, vref)
    else:
        P.kv_append(wl.new_k, wl.new_v, wl.slot_mapping.cuda(), kc, vc, km, vm)
        lens_after = wl.ctx_after.numpy()
        live = _live_slots(wl, lens_after)
        # oracle pools: its own quantisation of the live bf16 rows, the new tokens included
        kraw, vraw = wl.k_pool.clone(), wl.v_pool.clone()
        sl = wl.slot_mapping.cuda()
        kraw.view(NB * BS, H, D)[sl] = wl.new_k
        vraw.view(NB * BS, H, D)[sl] = wl.new_v
        raw = W.PagedWorkload(**{**wl.__dict__, "k_pool": kraw, "v_pool": vraw})
        kpool, vpool = _fp8_pools_oracle(raw, live)
        assert np.array_equal(kc.cpu().numpy()[live], kpool.cache[live])
        assert np.array_equal(vc.cpu().numpy()[live], vpool.cache[live])
    out = P.paged_decode(wl.q, kc, vc, wl.block_tables.cuda(), wl.ctx_after.cuda(), int(wl.ctx_after.max()),
                         wl.sm_scale, k_meta=km, v_meta=vm)
    want = paged_decode_ref(f32_of(wl.q), kpool, vpool, wl.block_tables.numpy(), wl.ctx_after.numpy(),
                            BS, H, wl.sm_scale)
    assert report(f"dual-stacked {kind}", f32_of(out), want, wl.dtype) <= ATTN_TOL


def test_max_batch_ragged():
    """The largest batch the ABI accepts (8192 requests): the per-workgroup prefix of context
    lengths is built over several passes of the workgroup's threads, and contexts of 0 and a
    few tokens are mixed; every row against the oracle."""
    P = need_gpu()
    B = 8192
    wl = W.decode_workload("max-batch", batch=B, num_q_heads=8, num_kv_heads=2, head_dim=64,
                           block_size=16, ctx_lo=0, ctx_hi=40, dtype=torch.float16, device="cuda",
                           seed=W.BASE_SEED + 61, append_one=False)
    assert int((wl.ctx_after == 0).sum()) > 0
    want = _oracle_same(wl, wl.k_pool, wl.v_pool, wl.ctx_after)
    for ps in (0, 32):
        out = _decode(P, wl, wl.k_pool, wl.v_pool, wl.ctx_after, partition_size=ps)
        got = f32_of(out)
        assert np.all(got[wl.ctx_after.numpy() == 0] == 0)
        assert report(f"max batch ps{ps}", got, want, wl.dtype) <= ATTN_TOL


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("D,bs", [(128, 16), (64, 64)])
def test_u3_decode_shapes_ragged(G, D, bs):
    """3-bit pools (quantised and packed by the oracle, uploaded as they are) at group sizes and
    head dims the full-size cases do not use; ragged and empty contexts, two partition sizes.
    With 2 kv heads a wave instruction holds tokens of 2 heads, so these run the row-major
    own-head form (its query-sum selection for 2 and 4 heads included); the matrix-core form at
    8 kv heads is covered in test_gpu_mq_shapes.py."""
    P = need_gpu()
    Hkv = 2
    lens = [1, 15, 16, 17, 511, 512, 513, 1000, 0, 33]
    wl = W.decode_workload("u3-ragged", batch=len(lens), num_q_heads=G * Hkv, num_kv_heads=Hkv,
                           head_dim=D, block_size=bs, ctx_lo=0, ctx_hi=0, dtype=torch.float16,
                           device="cuda", seed=300 + G + D + bs, append_one=False, ctx_override=lens,
                           poison=False)
    NB, BS, H, _ = wl.k_pool.shape
    slots = torch.arange(NB * BS, dtype=torch.int64)
    kpool, vpool = _u3_pools_from_raw(wl, wl.k_pool.reshape(NB * BS, H, D), wl.v_pool.reshape(NB * BS, H, D),
                                      slots)
    kc = torch.from_numpy(kpool.cache.view(np.int32)).cuda()
    vc = torch.from_numpy(vpool.cache.view(np.int32)).cuda()
    km = torch.from_numpy(kpool.meta).cuda()
    vm = torch.from_numpy(vpool.meta).cuda()
    want = paged_decode_ref(f32_of(wl.q), kpool, vpool, wl.block_tables.numpy(), np.array(lens), bs, Hkv,
                            wl.sm_scale)
    for ps in (0, 512):
        out = P.paged_decode(wl.q, kc, vc, wl.block_tables.cuda(), wl.ctx_after.cuda(), max(lens),
                             wl.sm_scale, k_meta=km, v_meta=vm, partition_size=ps, cache_dtype="u3")
        got = f32_of(out)
        assert np.all(got[lens.index(0)] == 0)
        assert report(f"u3 G{G} D{D} bs{bs} ps{ps}", got, want, torch.float16) <= ATTN_TOL

"""Pins of the slot_mapping builder and the append oracle, on the synthetic workloads.

Page: "Write Triton Kv Cache Append Kernel" - Inputs items 6-7 (paged slot id),
Required reasoning process steps 3, 5, 7, 9 (slot < 0 no-op, block/offset
decomposition, store, pre-increment decode position, prefill expansion),
Correctness requirements (readback through the slot mapping, padding leaves the
rest of the cache untouched, idempotence, GQA writes only kv heads), Common
failure modes (off-by-one positions, block index in physical units).
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_45_amd import workloads as W
from oracle import (decode_slot_mapping, prefill_slot_mapping, append_ref, CacheSpec,
                    paged_decode_ref, PoolView, quantize_fp8_rows, quantize_u3_rows,
                    quantize_e5m2_rows, quantize_int8_rows,
                    pack_rows_u3)
from oracle.append import to_f32


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


@pytest.mark.parametrize("maker", [W.tiny, W.llama8b_decode])
def test_decode_slots_agree_with_allocator(maker):
    wl = maker("cpu", make_pool=False) if maker is W.llama8b_decode else maker("cpu")
    got = decode_slot_mapping(wl.block_tables.numpy(), wl.ctx_before.numpy(), wl.block_size)
    assert np.array_equal(got, wl.slot_mapping.numpy())


def test_prefill_slots_agree_with_allocator():
    wl = W.mixed_append("cpu")
    pad = wl.token_request.numpy() < 0
    got = prefill_slot_mapping(wl.block_tables.numpy(), wl.req_start, wl.req_count,
                               wl.block_size, pad_mask=pad)
    assert np.array_equal(got, wl.slot_mapping.numpy())
    T = len(got)
    assert abs(pad.sum() - round(0.1 * T)) <= 1
    # a correct mapping never sends two tokens to one slot
    live = got[got >= 0]
    assert len(np.unique(live)) == len(live)


def test_off_by_one_mutations_are_caught():
    """Failure mode: using ctx-1 overwrites the previous token; ctx+1 leaves the new
    token's slot unwritten, so the decode then reads a poisoned slot."""
    wl = W.tiny("cpu")
    bt, ctx, BS = wl.block_tables.numpy(), wl.ctx_before.numpy(), wl.block_size
    kb, vb = _bits(wl.k_pool), _bits(wl.v_pool)
    nk, nv = _bits(wl.new_k), _bits(wl.new_v)
    spec = CacheSpec("same", "f16")

    def run(slots):
        k, v = kb.copy(), vb.copy()
        append_ref(nk, nv, slots, k, v, spec, BS)
        pools = (PoolView("same", k, dtype="f16"), PoolView("same", v, dtype="f16"))
        return paged_decode_ref(wl.q.float().numpy(), *pools, bt, wl.ctx_after.numpy(), BS,
                                wl.num_kv_heads, wl.sm_scale)

    good = run(decode_slot_mapping(bt, ctx, BS))
    assert np.all(np.isfinite(good))
    minus = run(decode_slot_mapping(bt, ctx - 1, BS))
    plus = run(decode_slot_mapping(bt, ctx + 1, BS))
    assert not np.all(np.isfinite(minus)) or np.max(np.abs(minus - good)) > 1e-3
    assert not np.all(np.isfinite(plus))


def test_append_readback_padding_untouched_idempotent():
    wl = W.mixed_append("cpu", num_prompts=2, prompt_lo=20, prompt_hi=70, num_decode=5,
                        ctx_lo=10, ctx_hi=90, block_size=16, head_dim=64, num_kv_heads=2)
    nb, BS, H, D = wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim
    rng = np.random.default_rng(0)
    k0 = rng.integers(0, 2 ** 16, (nb, BS, H, D), dtype=np.uint16)
    v0 = rng.integers(0, 2 ** 16, (nb, BS, H, D), dtype=np.uint16)
    k, v = k0.copy(), v0.copy()
    nk, nv = _bits(wl.new_k), _bits(wl.new_v)
    slots = wl.slot_mapping.numpy()
    append_ref(nk, nv, slots, k, v, CacheSpec("same", "bf16"), BS)
    written = np.zeros((nb, BS), dtype=bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), BS)
        written[blk, off] = True
        # readback: cache[slot] == new[token] (K and V separately, no cross-talk)
        assert np.array_equal(k[blk, off], nk[t]) and np.array_equal(v[blk, off], nv[t])
    # every slot that no valid token maps to is bit-identical to before
    assert np.array_equal(k[~written], k0[~written]) and np.array_equal(v[~written], v0[~written])
    # idempotence
    k2, v2 = k.copy(), v.copy()
    append_ref(nk, nv, slots, k2, v2, CacheSpec("same", "bf16"), BS)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    # out-of-range slots are skipped
    bad = slots.copy()
    bad[0] = nb * BS
    k3, v3 = k0.copy(), v0.copy()
    append_ref(nk[:1], nv[:1], bad[:1], k3, v3, CacheSpec("same", "bf16"), BS)
    assert np.array_equal(k3, k0)


@pytest.mark.parametrize("kind", ["fp8", "e5m2", "i8", "u3"])
def test_quantised_append_matches_row_quantiser(kind):
    wl = W.mixed_append("cpu", num_prompts=1, prompt_lo=40, prompt_hi=40, num_decode=3,
                        ctx_lo=5, ctx_hi=30, block_size=16, head_dim=128, num_kv_heads=2)
    nb, BS, H, D = wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim
    nk, nv = _bits(wl.new_k), _bits(wl.new_v)
    slots = wl.slot_mapping.numpy()
    if kind in ("fp8", "e5m2", "i8"):
        k = np.zeros((nb, BS, H, D), np.uint8)
        km = np.zeros((nb, BS, H), np.float32)
    else:
        k = np.zeros((nb, BS, H, D * 3 // 32), np.uint32)
        km = np.zeros((nb, BS, H, 2), np.float16)
    v, vm = k.copy(), km.copy()
    append_ref(nk, nv, slots, k, v, CacheSpec(kind, "bf16"), BS, km, vm)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), BS)
        x = to_f32(nk[t], "bf16")
        if kind == "fp8":
            codes, sc = quantize_fp8_rows(x)
            assert np.array_equal(k[blk, off], codes) and np.array_equal(km[blk, off], sc)
        elif kind in ("e5m2", "i8"):
            codes, sc = (quantize_e5m2_rows if kind == "e5m2" else quantize_int8_rows)(x)
            assert np.array_equal(k[blk, off], codes.view(np.uint8)) and np.array_equal(km[blk, off], sc)
        else:
            q, s16, z16 = quantize_u3_rows(x)
            assert np.array_equal(k[blk, off], pack_rows_u3(q))
            assert np.array_equal(km[blk, off, :, 0], s16) and np.array_equal(km[blk, off, :, 1], z16)


def test_workload_shapes():
    wl = W.llama8b_decode("cpu", make_pool=False)
    assert wl.batch == 64 and wl.group == 4 and wl.head_dim == 128 and wl.block_size == 16
    c = wl.ctx_before.numpy()
    assert c.min() >= 512 and c.max() <= 4096
    assert np.array_equal(wl.ctx_after.numpy(), c + 1)
    m = W.mixed_append("cpu")
    assert 4000 < m.slot_mapping.numel() < 17000 and m.block_size == 32
    lc = W.long_context("cpu", batch=2, ctx_lo=64, ctx_hi=200)
    assert lc.group == 8 and lc.block_size == 64


# ---- per-token slot ids from (request, position): the launcher's step, built on the device
# by build_slot_mapping ("Write Triton Kv Cache Append Kernel", Inputs items 6-7, step 9)

from oracle import slot_mapping_ref


def test_slot_mapping_ref_agrees_with_allocator_and_page_forms():
    wl = W.mixed_append("cpu")
    got = slot_mapping_ref(wl.token_request.numpy(), wl.token_position.numpy(), wl.block_tables.numpy(),
                           wl.block_size, len(wl.req_start))
    assert np.array_equal(got, wl.slot_mapping.numpy())
    d = W.llama8b_decode("cpu", make_pool=False)
    got = slot_mapping_ref(None, d.ctx_before.numpy(), d.block_tables.numpy(), d.block_size, d.batch)
    assert np.array_equal(got, d.slot_mapping.numpy())
    assert np.array_equal(got, decode_slot_mapping(d.block_tables.numpy(), d.ctx_before.numpy(),
                                                   d.block_size))


def test_slot_mapping_ref_worked_by_hand():
    bt = np.array([[7, 2, 0], [4, 9, 0]], np.int32)          # block size 16, 3 table entries
    req = np.array([0, 0, 1, 1, -1, 2, 0, 1], np.int64)
    pos = np.array([0, 17, 15, 31, 5, 0, 48, -1], np.int64)
    # 0 -> 7*16+0; 17 -> block 2, +1; 15 -> 4*16+15; 31 -> 9*16+15; padding; request 2 of 2;
    # position 48 = table entry 3 (outside the row); negative position
    assert slot_mapping_ref(req, pos, bt, 16, 2).tolist() == [112, 33, 79, 159, -1, -1, -1, -1]
    # contiguous cache, max_seq_len 64: r * 64 + p, positions >= 64 rejected
    pos2 = np.array([0, 17, 15, 63, 5, 0, 64, 3], np.int64)
    assert slot_mapping_ref(req, pos2, None, 64, 3).tolist() == [0, 17, 79, 127, -1, 128, -1, 67]


def test_contiguous_cache_through_the_paged_oracle():
    """The contiguous cache [B, Hkv, S, D] with slot r*S + p is the paged pool of block size S
    whose block r is request r, seen through the (request, position, head) transposed view:
    the oracle's append writes cache[r, h, p] = new[t, h], and its decode over that view equals
    its decode over a shuffled paged copy of the same rows."""
    B, H, S, D, BS = 3, 2, 64, 8, 16
    rng = np.random.default_rng(11)
    cache_k = np.zeros((B, H, S, D), np.uint16)
    cache_v = np.zeros((B, H, S, D), np.uint16)
    lens = [5, 64, 33]
    req = np.concatenate([np.full(n, r) for r, n in enumerate(lens)])
    pos = np.concatenate([np.arange(n) for n in lens])
    slots = slot_mapping_ref(req, pos, None, S, B)
    new_k = rng.integers(0x3C00, 0x4400, (len(req), H, D)).astype(np.uint16)   # fp16 in [1, 4)
    new_v = rng.integers(0xBC00, 0xC400, (len(req), H, D)).astype(np.uint16)
    view_k, view_v = cache_k.transpose(0, 2, 1, 3), cache_v.transpose(0, 2, 1, 3)
    append_ref(new_k, new_v, slots, view_k, view_v, CacheSpec("same", "f16"), S)
    for t in range(len(req)):
        assert np.array_equal(cache_k[req[t], :, pos[t]], new_k[t])
        assert np.array_equal(cache_v[req[t], :, pos[t]], new_v[t])
    q = rng.standard_normal((B, 4, D))
    want = paged_decode_ref(q, PoolView("same", view_k, dtype="f16"), PoolView("same", view_v, dtype="f16"),
                            np.arange(B).reshape(B, 1), np.array(lens), S, H, 0.3)
    # the same rows in a shuffled paged pool of 16-token blocks
    nblk = B * S // BS
    perm = rng.permutation(nblk)
    pk = np.zeros((nblk, BS, H, D), np.uint16)
    pv = pk.copy()
    bt = np.zeros((B, S // BS), np.int32)
    for r in range(B):
        for j in range(S // BS):
            blk = perm[r * (S // BS) + j]
            bt[r, j] = blk
            pk[blk] = view_k[r, j * BS:(j + 1) * BS]
            pv[blk] = view_v[r, j * BS:(j + 1) * BS]
    got = paged_decode_ref(q, PoolView("same", pk, dtype="f16"), PoolView("same", pv, dtype="f16"), bt,
                           np.array(lens), BS, H, 0.3)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_to_f32_matches_torch_on_every_16bit_pattern():
    """The oracle's widening of fp16 and bf16 bit patterns against torch's own conversions, on
    all 65,536 patterns of each (NaN patterns compared as NaN)."""
    import torch
    from oracle.append import to_f32
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for name, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        got = to_f32(bits, name)
        want = torch.from_numpy(bits.view(np.int16)).view(dt).to(torch.float32).numpy()
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), name
        assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32)), name

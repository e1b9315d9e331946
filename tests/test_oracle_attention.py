"""Pins of the paged decode attention oracle.

Page: "Triton KV Cache and PagedAttention" (llm-algo-leetcode ch. 10) - Step 1
(block pool and block table), the Step 4 test (dense reference built by gathering
blocks through the table, cutting to the context length and running per-head
softmax(q k^T * scale) v; tolerance 2e-3), the reference answer TODO 1-5 (table
lookup, masking, online softmax).  "Write Triton Kv Cache Append Kernel" -
Inputs item 3 and Kernel design rules (GQA by index arithmetic).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import paged_decode_ref, paged_decode_split_ref, lse_merge_ref, PoolView


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _scatter_dense(rng, K, V, block_size, num_blocks, dtype="f16"):
    """Scatter dense per-request K/V [L_b, Hkv, D] into a shuffled pool; return pool
    bits, block table and lens.  Unused slots/blocks hold NaN bits."""
    B = len(K)
    Hkv, D = K[0].shape[1], K[0].shape[2]
    nan = 0x7E00 if dtype == "f16" else 0x7FC0
    kp = np.full((num_blocks, block_size, Hkv, D), nan, dtype=np.uint16)
    vp = kp.copy()
    need = [-(-k.shape[0] // block_size) for k in K]
    perm = rng.permutation(num_blocks)
    bt = np.zeros((B, max(max(need), 1)), dtype=np.int32)
    off = 0
    for b in range(B):
        blks = perm[off:off + need[b]]
        off += need[b]
        bt[b, :need[b]] = blks
        for t in range(K[b].shape[0]):
            kp[blks[t // block_size], t % block_size] = K[b][t]
            vp[blks[t // block_size], t % block_size] = V[b][t]
    return kp, vp, bt


def _f16_bits(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def _sdpa_dense(q, K, V, sm_scale, G):
    """torch float64 SDPA on dense tensors with K/V repeated by G (library routine)."""
    out = []
    for b in range(len(K)):
        if K[b].shape[0] == 0:
            out.append(np.zeros(q[b].shape))
            continue
        kk = torch.from_numpy(K[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
        vv = torch.from_numpy(V[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
        qq = torch.from_numpy(q[b].astype(np.float64))[:, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk.contiguous(), vv.contiguous(),
                                                             scale=sm_scale)
        out.append(o[:, 0, :].numpy())
    return np.stack(out)


def _case(seed, lens, Hq, Hkv, D, BS, spare=3):
    rng = np.random.default_rng(seed)
    K = [rng.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
    V = [rng.standard_normal((L, Hkv, D)).astype(np.float16) for L in lens]
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float16)
    nb = sum(-(-L // BS) for L in lens) + spare
    kp, vp, bt = _scatter_dense(rng, [_f16_bits(k) for k in K], [_f16_bits(v) for v in V], BS, nb)
    return q, K, V, kp, vp, bt, np.array(lens, dtype=np.int32)


def _ref(q, kp, vp, bt, lens, BS, Hkv, sm, dtype="f16", **kw):
    return paged_decode_ref(q, PoolView("same", kp, dtype=dtype), PoolView("same", vp, dtype=dtype),
                            bt, lens, BS, Hkv, sm, **kw)


def _bf16_case(seed, lens, Hq, Hkv, D, BS, spare=3):
    """The bf16 form of _case: values rounded to bf16 by torch's own cast (not the oracle's
    widening), bit patterns from torch, the dense side in float64 from the same bf16 values."""
    rng = np.random.default_rng(seed)
    gen = lambda shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    K = [gen((L, Hkv, D)) for L in lens]
    V = [gen((L, Hkv, D)) for L in lens]
    q = gen((len(lens), Hq, D))
    nb = sum(-(-L // BS) for L in lens) + spare
    kp, vp, bt = _scatter_dense(rng, [_bits(k) for k in K], [_bits(v) for v in V], BS, nb, dtype="bf16")
    f64 = lambda t: t.to(torch.float64).numpy()
    return (f64(q), [f64(k) for k in K], [f64(v) for v in V], kp, vp, bt,
            np.array(lens, dtype=np.int32))


@pytest.mark.parametrize("lens,Hq,Hkv,D,BS", [
    ([11, 26], 4, 4, 64, 16),
    ([1, 17, 33, 64], 8, 2, 64, 16),
    ([100, 5], 8, 1, 128, 32),
    ([200], 32, 8, 128, 64),
])
def test_brute_force_dense_sdpa(lens, Hq, Hkv, D, BS):
    q, K, V, kp, vp, bt, L = _case(3, lens, Hq, Hkv, D, BS)
    sm = 1.0 / math.sqrt(D)
    got = _ref(q, kp, vp, bt, L, BS, Hkv, sm)
    want = _sdpa_dense(q, K, V, sm, Hq // Hkv)
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("lens,Hq,Hkv,D,BS", [
    ([11, 26], 4, 4, 64, 16),
    ([1, 17, 33, 64], 8, 2, 64, 16),
    ([513, 100], 32, 8, 128, 16),
    ([200], 64, 8, 128, 64),
])
def test_brute_force_dense_sdpa_bf16(lens, Hq, Hkv, D, BS):
    """bf16 pools (the Llama-8B and long-context dtype) against torch's float64 SDPA on the
    same bf16 values, the pools' bit patterns written by torch's bf16 cast."""
    q, K, V, kp, vp, bt, L = _bf16_case(5, lens, Hq, Hkv, D, BS)
    sm = 1.0 / math.sqrt(D)
    got = _ref(q, kp, vp, bt, L, BS, Hkv, sm, dtype="bf16")
    want = _sdpa_dense(q, K, V, sm, Hq // Hkv)
    assert np.max(np.abs(got - want)) < 1e-12


def test_literal_tiny_case_from_page(golden_dir):
    """The page's own tiny check: literal block table, context lengths 10 and 25."""
    cfg = json.load(open(os.path.join(golden_dir, "paged_tiny_case.json")))
    rng = np.random.default_rng(cfg["seed"])
    NB, BS, H, D = cfg["num_blocks"], cfg["block_size"], cfg["num_heads"], cfg["head_dim"]
    kp = _f16_bits(rng.standard_normal((NB, BS, H, D)))
    vp = _f16_bits(rng.standard_normal((NB, BS, H, D)))
    q = rng.standard_normal((cfg["batch"], H, D)).astype(np.float16)
    bt = np.array(cfg["block_tables"], dtype=np.int32)
    L = np.array(cfg["context_lens"], dtype=np.int32)
    got = _ref(q, kp, vp, bt, L, BS, H, cfg["sm_scale"])
    # the page's dense construction: concatenate the table's blocks, cut to length
    K = [np.concatenate([kp[bt[b, i]] for i in range(math.ceil(L[b] / BS))])[:L[b]].view(np.float16)
         for b in range(2)]
    V = [np.concatenate([vp[bt[b, i]] for i in range(math.ceil(L[b] / BS))])[:L[b]].view(np.float16)
         for b in range(2)]
    want = _sdpa_dense(q, K, V, cfg["sm_scale"], 1)
    assert np.max(np.abs(got - want)) < 1e-12


def test_block_permutation_invariance():
    q, K, V, kp, vp, bt, L = _case(5, [40, 70], 4, 2, 64, 16, spare=6)
    base = _ref(q, kp, vp, bt, L, 16, 2, 0.125)
    perm = np.random.default_rng(1).permutation(kp.shape[0])
    inv = np.argsort(perm)
    kp2, vp2 = kp[perm], vp[perm]             # block i moves to position inv[i]
    bt2 = inv[bt].astype(np.int32)
    assert np.max(np.abs(_ref(q, kp2, vp2, bt2, L, 16, 2, 0.125) - base)) < 1e-12


def test_single_token_returns_v0_and_equal_keys_return_mean():
    q, K, V, kp, vp, bt, L = _case(6, [1, 30], 2, 2, 64, 16)
    out = _ref(q, kp, vp, bt, L, 16, 2, 0.125)
    assert np.allclose(out[0], V[0][0].astype(np.float64), atol=0, rtol=0)
    # equal keys: every token of request 1 gets the same key -> uniform weights
    kp2 = kp.copy()
    for t in range(30):
        kp2[bt[1, t // 16], t % 16] = kp[bt[1, 0], 0]
    out2 = _ref(q, kp2, vp, bt, L, 16, 2, 0.125)
    assert np.max(np.abs(out2[1] - V[1].astype(np.float64).mean(axis=0))) < 1e-12


def test_gqa_equals_mha_on_repeated_kv():
    Hq, Hkv, D = 8, 2, 64
    q, K, V, kp, vp, bt, L = _case(7, [23, 50], Hq, Hkv, D, 16)
    gqa = _ref(q, kp, vp, bt, L, 16, Hkv, 0.125)
    G = Hq // Hkv
    kp_rep, vp_rep = np.repeat(kp, G, axis=2), np.repeat(vp, G, axis=2)
    mha = _ref(q, kp_rep, vp_rep, bt, L, 16, Hq, 0.125)
    assert np.max(np.abs(gqa - mha)) < 1e-12
    # the plausible mistake h % Hkv instead of h // G gives a different answer
    wrong = np.stack([mha[:, (h % Hkv) * G + (h // Hkv)] for h in range(Hq)], axis=1)
    assert np.max(np.abs(wrong - gqa)) > 1e-3


def test_poisoned_slots_never_reach_output():
    q, K, V, kp, vp, bt, L = _case(8, [17, 31], 4, 4, 64, 16)
    out = _ref(q, kp, vp, bt, L, 16, 4, 0.125)
    assert np.isnan(kp.view(np.float16)).any() and np.isnan(vp.view(np.float16)).any()
    assert np.all(np.isfinite(out))


def test_zero_length_gives_zero():
    q, K, V, kp, vp, bt, L = _case(9, [0, 5], 4, 4, 64, 16)
    out = _ref(q, kp, vp, bt, L, 16, 4, 0.125)
    assert np.all(out[0] == 0)


@pytest.mark.parametrize("P", [16, 64, 512, 4096])
def test_split_equals_single_pass(P):
    q, K, V, kp, vp, bt, L = _case(10, [1, 100, 777, 1500], 8, 2, 64, 16)
    pools = (PoolView("same", kp, dtype="f16"), PoolView("same", vp, dtype="f16"))
    one = paged_decode_ref(q, *pools, bt, L, 16, 2, 0.125)
    split = paged_decode_split_ref(q, *pools, bt, L, 16, 2, 0.125, P)
    assert np.max(np.abs(one - split)) < 1e-12


def test_lse_merge_closed_form_and_empty_partitions():
    rng = np.random.default_rng(11)
    s = rng.standard_normal(50) * 3
    v = rng.standard_normal((50, 8))
    p = np.exp(s - s.max())
    want = p @ v / p.sum()
    parts = [(0, 20), (20, 21), (21, 50)]
    m = np.array([s[a:b].max() for a, b in parts] + [-np.inf])
    l = np.array([np.exp(s[a:b] - s[a:b].max()).sum() for a, b in parts] + [0.0])
    acc = np.array([np.exp(s[a:b] - s[a:b].max()) @ v[a:b] for a, b in parts] + [np.zeros(8)])
    assert np.max(np.abs(lse_merge_ref(m, l, acc) - want)) < 1e-12


def test_mutations_fail_brute_force():
    """Plausible oracle mistakes that the dense brute force must reject."""
    q, K, V, kp, vp, bt, L = _case(12, [40, 70], 4, 4, 64, 16)
    want = _sdpa_dense(q, K, V, 0.125, 1)
    good = _ref(q, kp, vp, bt, L, 16, 4, 0.125)
    assert np.max(np.abs(good - want)) < 1e-12
    # (a) scale dropped
    assert np.max(np.abs(_ref(q, kp, vp, bt, L, 16, 4, 1.0) - want)) > 1e-3
    # (b) one token too many (off-by-one in the mask) reads a NaN-poisoned slot
    bad = _ref(q, kp, vp, bt, L + 1, 16, 4, 0.125)
    assert not np.all(np.isfinite(bad)) or np.max(np.abs(bad - want)) > 1e-3
    # (c) K and V swapped
    assert np.max(np.abs(_ref(q, vp, kp, bt, L, 16, 4, 0.125) - want)) > 1e-3

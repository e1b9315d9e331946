"""GPU parity of pack3 / unpack3 against the oracle, bit-exact.

"triton-3bit-kv-cache-kernel" README, section 2 test 1 (and test 5A on its GPU): every
one of the 2^24 octet states, both inverses; section 2 test 2: walking patterns.
"""
import time

import numpy as np
import pytest
import torch

from gpu_helpers import need_gpu
import oracle

pytestmark = pytest.mark.gpu


def _all_octet_values():
    i = np.arange(1 << 24, dtype=np.uint32)
    return np.stack([(i >> np.uint32(3 * j)) & np.uint32(7) for j in range(8)], axis=1).astype(np.uint8).reshape(-1)


def _all_byte_triples():
    i = np.arange(1 << 24, dtype=np.uint32)
    return np.stack([(i >> np.uint32(8 * k)) & np.uint32(255) for k in range(3)], axis=1).astype(np.uint8).reshape(-1)


def test_exhaustive_2pow24_both_inverses():
    P = need_gpu()
    vals = _all_octet_values()
    trip = _all_byte_triples()
    want_packed = oracle.pack3(vals)
    want_vals = oracle.unpack3(trip)
    dv = torch.from_numpy(vals).cuda()
    dt = torch.from_numpy(trip).cuda()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    packed = P.pack3(dv)
    back = P.unpack3(packed, dv.numel())
    unpacked = P.unpack3(dt)
    repacked = P.pack3(unpacked)
    torch.cuda.synchronize()
    dt_ms = (time.perf_counter() - t0) * 1e3
    assert np.array_equal(packed.cpu().numpy(), want_packed)
    assert np.array_equal(back.cpu().numpy(), vals)                 # left inverse
    assert np.array_equal(unpacked.cpu().numpy(), want_vals)
    assert np.array_equal(repacked.cpu().numpy(), trip)             # right inverse
    print(f"exhaustive 2^24 pack3+unpack3 both ways on GPU: {dt_ms:.2f} ms (incl. launches)", flush=True)


@pytest.mark.parametrize("n_values,offset_v,offset_p", [
    (8, 0, 0), (40, 0, 0), (32 * 1000 + 24, 0, 0), (4096, 1, 0), (4096, 0, 1), (1000 * 8, 3, 5)])
def test_ragged_tails_and_unaligned(n_values, offset_v, offset_p):
    P = need_gpu()
    rng = np.random.default_rng(n_values + offset_v)
    vals = rng.integers(0, 256, n_values, dtype=np.uint8)         # high bits must be ignored
    bufv = torch.zeros(n_values + 16, dtype=torch.uint8, device="cuda")
    bufp = torch.full((3 * n_values // 8 + 16,), 0xAB, dtype=torch.uint8, device="cuda")
    dv = bufv[offset_v:offset_v + n_values]
    dv.copy_(torch.from_numpy(vals))
    dp = bufp[offset_p:offset_p + 3 * n_values // 8]
    P.pack3(dv, dp)
    want = oracle.pack3(vals)
    host = bufp.cpu().numpy()
    assert np.array_equal(host[offset_p:offset_p + want.size], want)
    assert np.all(host[:offset_p] == 0xAB) and np.all(host[offset_p + want.size:] == 0xAB)
    out = torch.full((n_values + 16,), 0xCD, dtype=torch.uint8, device="cuda")
    P.unpack3(dp, n_values, out[offset_v:offset_v + n_values])
    oh = out.cpu().numpy()
    assert np.array_equal(oh[offset_v:offset_v + n_values], vals & 7)
    assert np.all(oh[offset_v + n_values:] == 0xCD)


def test_walking_patterns_on_gpu():
    P = need_gpu()
    rows = []
    for bg in (0, 7):
        for lane in range(32):
            for v in range(8):
                r = np.full(32, bg, dtype=np.uint8)
                r[lane] = v
                rows.append(r)
    vals = np.concatenate(rows)
    packed = P.pack3(torch.from_numpy(vals).cuda()).cpu().numpy()
    want = np.concatenate([oracle.pack3_words(r).view(np.uint8) for r in rows])
    assert np.array_equal(packed, want)
    assert np.array_equal(P.unpack3(torch.from_numpy(packed).cuda()).cpu().numpy(), vals)


def test_empty_and_invalid_sizes():
    P = need_gpu()
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    assert P.pack3(e).numel() == 0
    with pytest.raises(P.PagedKVError):
        P.pack3(torch.zeros(12, dtype=torch.uint8, device="cuda"))

"""Pins of the e5m2 and int8 cache quantisers of the oracle.

Page: "Write Triton Kv Cache Append Kernel" - Inputs item 4 (fp8 or int8 caches with fp32
scales), Required reasoning process step 6 (divide by the scale in fp32, then cast; fp8 may
be e4m3 or e5m2), Correctness requirements (the dequantised cache is within one quantisation
step).  Library special cases: torch's float8_e5m2 dtype (decode of every code, and its CPU
cast, which rounds to nearest even inside the finite range).  Closed form: an e5m2 code is
the upper byte of the fp16 encoding of the same value, so rounding an fp16 value to e5m2 is
round-to-nearest-even of its fp16 bits at bit 8.
"""
import numpy as np
import pytest
import torch

from oracle import (e5m2_decode_table, e5m2_decode, e5m2_encode_rne, quantize_e5m2_rows,
                    quantize_int8_rows, dequantize_e5m2_rows, dequantize_int8_rows, E5M2_MAX,
                    INT8_MAX)


def _torch_e5m2_codes(y):
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e5m2) \
        .view(torch.uint8).numpy()


def test_e5m2_decode_table_matches_torch_and_definition():
    mine = e5m2_decode_table()
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(theirs))
    ok = ~np.isnan(mine)
    assert np.array_equal(mine[ok], theirs[ok])
    assert mine[0x7B] == E5M2_MAX == 57344.0
    assert mine[0x7C] == np.inf and mine[0xFC] == -np.inf
    assert np.nonzero(np.isnan(mine))[0].tolist() == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    assert mine[0x01] == 2.0 ** -16 and mine[0x04] == 2.0 ** -14      # subnormal, smallest normal
    # every code is the upper byte of the fp16 value it denotes
    as_f16 = (np.arange(256, dtype=np.uint16) << np.uint16(8)).view(np.float16).astype(np.float64)
    assert np.array_equal(as_f16[ok], mine[ok])


def test_e5m2_encoder_on_every_fp16_value_closed_form():
    """All finite fp16 values with |y| <= 57344: the code is the fp16 bit pattern rounded to
    nearest even at bit 8 (sign handled apart, the carry runs into the exponent)."""
    h = np.arange(0x8000, dtype=np.uint32)
    y16 = h.astype(np.uint16).view(np.float16)
    keep = np.isfinite(y16) & (np.abs(y16.astype(np.float32)) <= E5M2_MAX)
    h, y16 = h[keep], y16[keep]
    want = ((h + 0x7F + ((h >> 8) & 1)) >> 8).astype(np.uint8)
    for sign in (1.0, -1.0):
        y = (y16.astype(np.float32) * np.float32(sign))
        got = e5m2_encode_rne(y)
        exp = want | (np.uint8(0x80) if sign < 0 else np.uint8(0))
        assert np.array_equal(got, exp)


def _grid_probe_values():
    """Every finite e5m2 value, every midpoint between neighbours, and 4 fp32 ulps either side
    of each of them, both signs."""
    vals = e5m2_decode_table()[:0x7C]
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    out = [pts]
    up, down = pts.copy(), pts.copy()
    for _ in range(4):
        up = np.nextafter(up, np.float32(np.inf))
        down = np.nextafter(down, np.float32(-np.inf))
        out += [up, down]
    y = np.concatenate(out)
    y = y[(y >= 0) & (y <= E5M2_MAX)]
    return np.concatenate([y, -y])


def test_e5m2_encoder_vs_torch_near_grid_and_strided():
    y = _grid_probe_values()
    assert np.array_equal(e5m2_encode_rne(y), _torch_e5m2_codes(y))
    # a strided sweep over every fp32 bit pattern up to 57344, both signs
    bits = np.arange(0, 0x47600001, 1201, dtype=np.uint32)
    for sign in (0, 0x80000000):
        ys = (bits + np.uint32(sign)).view(np.float32)
        assert np.array_equal(e5m2_encode_rne(ys), _torch_e5m2_codes(ys))


def test_e5m2_encoder_brute_force_tiny():
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.uniform(-4, 4, 300), rng.uniform(-1e-4, 1e-4, 300),
                        rng.uniform(-E5M2_MAX, E5M2_MAX, 300)]).astype(np.float32)
    table = e5m2_decode_table()
    codes = np.arange(256)
    fin = np.isfinite(table)
    got = e5m2_encode_rne(y)
    for v, g in zip(y.astype(np.float64), got):
        d = np.abs(table[fin] - v)
        best = codes[fin][d == d.min()]
        best = [c for c in best if (c >> 7) == int(np.signbit(v))] or list(best)
        even = [c for c in best if c % 2 == 0]
        assert g == (even[0] if even else best[0])


def test_e5m2_rows_and_round_trip_bound():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 128)).astype(np.float32) * np.float32(3.0)
    x[3] = 0.0
    codes, s = quantize_e5m2_rows(x)
    assert s[3] == 1.0 and np.all(codes[3] == 0)
    absmax = np.abs(x).max(axis=1)
    # the largest element lands on the top of the range
    i = np.arange(64) != 3
    top = e5m2_decode(codes[i, np.abs(x[i]).argmax(axis=1)])
    assert np.all(np.abs(top) == E5M2_MAX)
    # one step: |x - decode * s| <= half the quantum of x's binade (relative 2^-3) plus the
    # fp32 division's rounding
    back = dequantize_e5m2_rows(codes, s)
    y = np.abs(x.astype(np.float64) / s[:, None])
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -14)))
    half_q = 2.0 ** (e - 3) * s[:, None]
    assert np.all(np.abs(back - x) <= half_q * (1 + 1e-6) + 1e-30)
    assert np.all(np.abs(back[i] - x[i]).max(axis=1) <= absmax[i] / 8)


def test_int8_rows_worked_by_hand():
    # absmax 127 -> s = 1: the codes are x rounded half to even
    x = np.array([[127.0, 63.5, -63.5, 0.5, -1.5, 2.5, -127.0, 0.49]], np.float32)
    codes, s = quantize_int8_rows(x)
    assert s.tolist() == [1.0]
    assert codes.tolist() == [[127, 64, -64, 0, -2, 2, -127, 0]]
    # absmax 254 -> s = 2: 3.0 / 2 = 1.5 -> 2, 5.0 / 2 = 2.5 -> 2, -254 -> -127
    x = np.array([[254.0, 3.0, 5.0, -254.0, 1.0]], np.float32)
    codes, s = quantize_int8_rows(x)
    assert s.tolist() == [2.0] and codes.tolist() == [[127, 2, 2, -127, 0]]
    codes, s = quantize_int8_rows(np.zeros((2, 8), np.float32))
    assert s.tolist() == [1.0, 1.0] and np.all(codes == 0)
    assert dequantize_int8_rows(np.array([[0x81, 0x7F, 0xFF]], np.uint8), np.array([0.5])).tolist() \
        == [[-63.5, 63.5, -0.5]]


def test_int8_round_trip_bound_and_symmetry():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((256, 64)).astype(np.float32)
    codes, s = quantize_int8_rows(x)
    assert codes.min() >= -INT8_MAX and codes.max() <= INT8_MAX
    assert np.all(np.abs(codes).max(axis=1) == INT8_MAX)
    back = dequantize_int8_rows(codes, s)
    assert np.all(np.abs(back - x) <= s[:, None] * (0.5 + 1e-5))
    neg, _ = quantize_int8_rows(-x)
    assert np.array_equal(neg, -codes)


@pytest.mark.parametrize("bad", [E5M2_MAX * 1.01, np.inf, np.nan])
def test_e5m2_encoder_rejects_unclamped(bad):
    with pytest.raises(ValueError):
        e5m2_encode_rne(np.array([1.0, bad], np.float32))

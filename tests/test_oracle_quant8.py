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


# ---- caller-given scales (per-tensor / per-head / per-block / per-token granularity)

from oracle import (quantize_given_scale, scale_offsets, quantize_fp8_rows, append_ref, CacheSpec,
                    PoolView)

_ROW_QUANT = {"fp8": quantize_fp8_rows, "e5m2": quantize_e5m2_rows, "i8": quantize_int8_rows}


@pytest.mark.parametrize("kind", ["fp8", "e5m2", "i8"])
def test_given_scale_equal_to_row_scale_reduces_to_row_quantiser(kind):
    rng = np.random.default_rng(8)
    x = rng.standard_normal((50, 64)).astype(np.float32) * np.float32(2.5)
    codes, s = _ROW_QUANT[kind](x)
    assert np.array_equal(quantize_given_scale(x, s, kind), np.asarray(codes).view(np.uint8))


def test_given_scale_worked_by_hand():
    # s = 0.5: y = [2, -1.5, 600 (clamped), 0]
    x = np.array([[1.0, -0.75, 300.0, 0.0]], np.float32)
    s = np.array([0.5], np.float32)
    # e4m3fn: 2 = 2^1 -> exponent field 8; -1.5 -> field 7, mantissa 4; 448 = 0x7E
    assert quantize_given_scale(x, s, "fp8").tolist() == [[0x40, 0xBC, 0x7E, 0x00]]
    # e5m2: 2 -> field 16; -1.5 -> field 15, mantissa 2; 600 clamps nowhere (< 57344) and
    # rounds to 640 = 1.25 * 2^9 -> field 24, mantissa 1
    assert quantize_given_scale(x, s, "e5m2").tolist() == [[0x40, 0xBE, 0x61, 0x00]]
    # int8: -1.5 ties to -2; 600 saturates at 127
    assert quantize_given_scale(x, s, "i8").view(np.int8).tolist() == [[2, -2, 127, 0]]
    # e4m3fn saturation on the negative side
    assert quantize_given_scale(np.array([[-1e6]], np.float32), s, "fp8").tolist() == [[0xFE]]


@pytest.mark.parametrize("bad", [0.0, -1.0, np.inf, np.nan])
def test_given_scale_rejects_bad_scales(bad):
    with pytest.raises(ValueError):
        quantize_given_scale(np.ones((1, 8), np.float32), np.array([bad], np.float32), "i8")


@pytest.mark.parametrize("gran", ["tensor", "head", "block", "block_head", "token_head"])
@pytest.mark.parametrize("kind", ["fp8", "e5m2", "i8"])
def test_append_with_given_scales_reads_the_right_scale(gran, kind):
    """Tiny pool, distinct scales per granule: every written row decodes within half a step of
    its input under the scale its granule names, and the scale arrays are never written."""
    NB, BS, H, D = 3, 4, 2, 8
    strides = {"tensor": (0, 0, 0), "head": (0, 0, 1), "block": (1, 0, 0),
               "block_head": (H, 0, 1), "token_head": (BS * H, H, 1)}[gran]
    n_scales = {"tensor": 1, "head": H, "block": NB, "block_head": NB * H, "token_head": NB * BS * H}[gran]
    rng = np.random.default_rng(9)
    top = {"fp8": 448.0, "e5m2": 57344.0, "i8": 127.0}[kind]
    # |x| < 3, so every y = x / s stays inside the format's range (saturation is pinned above)
    scales = (rng.uniform(1.0, 2.0, n_scales) * 3.0 / top).astype(np.float32)
    T = 7
    x = rng.uniform(-3, 3, (T, H, D)).astype(np.float32)
    bits = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)     # bf16 (truncated)
    slots = np.array([0, 5, -1, 11, 6, 3, 9], np.int64)
    kc = np.zeros((NB, BS, H, D), np.uint8)
    vc = kc.copy()
    ks, vs = scales.copy(), scales.copy()
    append_ref(bits, bits, slots, kc, vc, CacheSpec(kind, "bf16"), BS, ks, vs, scale_strides=strides)
    assert np.array_equal(ks, scales) and np.array_equal(vs, scales)
    pool = PoolView(kind, kc, ks, scale_strides=strides)
    xb = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), BS)
        for h in range(H):
            s = float(scales[scale_offsets(blk, off, h, strides)])
            back = pool.rows(np.array([blk]), h)[off]
            y = np.abs(xb[t, h] / s)
            if kind == "i8":
                step = np.full_like(y, 1.0)
            else:
                man = 3 if kind == "fp8" else 2
                emin = -6 if kind == "fp8" else -14
                step = 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** emin))) - man)
            assert np.all(np.abs(back - xb[t, h]) <= step * s / 2 * (1 + 1e-6)), (gran, t, h)
    # untouched slots stay zero
    written = {int(v) for v in slots if v >= 0}
    for slot in range(NB * BS):
        if slot not in written:
            assert not kc[divmod(slot, BS)].any()

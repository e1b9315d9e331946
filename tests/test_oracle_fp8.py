"""Pins of the fp8 e4m3fn oracle.

Page: "Write Triton Kv Cache Append Kernel" - Inputs items 4 and 8 (fp8 cache with
an fp32 scale), Required reasoning process step 6 (divide by the scale in fp32,
then cast to float8e4nv, i.e. OCP E4M3), Correctness requirements (dequantised
cache within one quantisation step), Common failure modes (casting before scaling
loses range).  Library special case: torch's CPU float8_e4m3fn cast, which rounds
to nearest-even inside the finite range.
"""
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

from oracle import (e4m3fn_decode_table, e4m3fn_encode_rne, e4m3fn_decode, quantize_fp8_rows,
                    dequantize_fp8_rows, E4M3_MAX)

CHUNK = 1 << 23


def _torch_codes(y):
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch():
    mine = e4m3fn_decode_table()
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(theirs))
    ok = ~np.isnan(mine)
    assert np.array_equal(mine[ok], theirs[ok])
    assert np.nonzero(np.isnan(mine))[0].tolist() == [0x7F, 0xFF]
    assert mine[0x7E] == E4M3_MAX == 448.0
    assert mine[0x01] == 2.0 ** -9                      # smallest subnormal


def test_encoder_exhaustive_vs_torch():
    """Every fp32 bit pattern from 2^-11 up to 448, both signs (the range in which the
    code is not trivially zero), plus a strided sweep below 2^-11."""
    lo, hi = 0x3A000000, 0x43E00000 + 1                    # 2^-11 .. 448 inclusive
    ranges = []
    for sign in (0, 0x80000000):
        for a in range(lo, hi, CHUNK):
            ranges.append((sign + a, sign + min(a + CHUNK, hi)))
    import fp8_sweep_worker
    workers = max(1, min(8, os.cpu_count() or 1))
    # spawn, not fork: forking after torch has started its thread pools can deadlock
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        results = list(ex.map(fp8_sweep_worker.check_range, ranges))
    assert all(n == 0 for n, _ in results), [r for r in results if r[0]]
    # below 2^-11 every value rounds to (signed) zero; sweep with a prime stride
    bits = np.arange(0, lo, 9973, dtype=np.uint32)
    for sign in (0, 0x80000000):
        y = (bits + np.uint32(sign)).view(np.float32)
        assert np.array_equal(e4m3fn_encode_rne(y), _torch_codes(y))


def _brute_force_codes(y):
    """Nearest finite e4m3fn value by search over the table; ties to the even code."""
    table = e4m3fn_decode_table()
    codes = np.arange(256)
    finite = ~np.isnan(table)
    cand_codes = codes[finite]
    cand_vals = table[finite]
    out = np.empty(y.shape, dtype=np.uint8)
    for i, v in enumerate(y.astype(np.float64)):
        d = np.abs(cand_vals - v)
        best = d.min()
        tie = cand_codes[d == best]
        # among equally near codes keep those with the same sign as v (matters for 0)
        same_sign = [c for c in tie if (c >> 7) == (1 if np.signbit(v) else 0)]
        tie = np.array(same_sign if same_sign else tie)
        even = tie[(tie & 1) == 0]
        out[i] = even[0] if even.size else tie[0]
    return out


def test_encoder_brute_force_including_ties():
    rng = np.random.default_rng(1234)
    table = e4m3fn_decode_table()
    pos = np.sort(table[(~np.isnan(table)) & (table >= 0)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)        # exact ties
    rand = (rng.uniform(-448, 448, 4000)).astype(np.float32)
    small = (rng.uniform(-2 ** -5, 2 ** -5, 2000)).astype(np.float32)
    y = np.concatenate([mids, -mids, rand, small, pos.astype(np.float32), np.float32([-0.0])])
    assert np.array_equal(e4m3fn_encode_rne(y), _brute_force_codes(y))


def test_round_trip_within_half_step():
    """Correctness requirements: dequantised values within one quantisation step."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((256, 8, 128)).astype(np.float32) * rng.uniform(1e-3, 1e3, (256, 8, 1)).astype(np.float32)
    codes, s = quantize_fp8_rows(x)
    xhat = dequantize_fp8_rows(codes, s)
    y = np.abs(x.astype(np.float64) / s[..., None])
    _, fe = np.frexp(y)
    ulp = np.ldexp(1.0, np.maximum(fe - 1, -6) - 3)
    assert np.all(np.abs(x - xhat) <= 0.5 * ulp * s[..., None] * (1 + 1e-6) + 1e-30)
    # the largest magnitude of each row lands on +-448
    amax = np.abs(x).argmax(axis=-1)
    top = np.take_along_axis(codes, amax[..., None], axis=-1)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)


def test_zero_row_and_signed_zero():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 3] = -0.0
    codes, s = quantize_fp8_rows(x)
    assert np.all(s == 1.0)
    assert codes[0].tolist() == [0] * 64
    assert codes[1, 3] == 0x80


def test_cast_before_scale_is_a_different_result():
    """Common failure modes: casting to fp8 before dividing by the scale saturates."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((16, 128)) * 1000).astype(np.float32)
    codes, s = quantize_fp8_rows(x)
    wrong = e4m3fn_encode_rne(np.clip(x, -448, 448)).astype(np.float64)
    wrong_deq = e4m3fn_decode(wrong.astype(np.uint8)) / 1.0
    right_deq = dequantize_fp8_rows(codes, s)
    assert np.max(np.abs(right_deq - x)) < np.max(np.abs(wrong_deq - x)) / 10


def test_encoder_rejects_unclamped_input():
    with pytest.raises(ValueError):
        e4m3fn_encode_rne(np.float32([449.0]))

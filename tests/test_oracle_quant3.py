"""Pins of the 3-bit affine quantiser.

Page: "triton-3bit-kv-cache-kernel" README - title paragraph (uint3 codes 0..7,
register-level affine dequantisation) and section 2, test 3 (fp16 affine
dequant x_hat = (q - z) * s; requantising x_hat gives q back for every q in
0..7, on (64, 128) KV tiles).
"""
import numpy as np
import pytest

from oracle import quantize_u3_rows, dequantize_u3_rows


def _tiles(seed, shape=(64, 128), scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_requant_round_trip_all_codes(seed):
    """Section 2 test 3 on seeded (64, 128) tiles, in fp32 and in fp64."""
    x = _tiles(seed, scale=10.0 ** (seed - 1))
    _, s16, z16 = quantize_u3_rows(x)
    s32 = s16.astype(np.float32)[:, None]
    z32 = z16.astype(np.float32)[:, None]
    for qv in range(8):
        q = np.full(x.shape, qv, dtype=np.float32)
        xhat32 = ((q - z32) * s32).astype(np.float32)
        back32 = np.clip(np.rint((xhat32 / s32).astype(np.float32) + z32), 0, 7)
        assert np.array_equal(back32, q)
        xhat64 = dequantize_u3_rows(q.astype(np.uint8), s16, z16)
        back64 = np.clip(np.rint(xhat64 / s32.astype(np.float64) + z32.astype(np.float64)), 0, 7)
        assert np.array_equal(back64, q)


@pytest.mark.parametrize("seed", [10, 11])
def test_codes_in_range_and_grid_bound(seed):
    x = _tiles(seed, shape=(512, 128))
    q, s16, z16 = quantize_u3_rows(x)
    assert q.dtype == np.uint8 and q.max() <= 7
    xhat = dequantize_u3_rows(q, s16, z16)
    s = s16.astype(np.float64)[:, None]
    # half a grid step, plus what fp16 rounding of s and z can shift the grid by
    z = z16.astype(np.float64)[:, None]
    slack = s * (7 * 2.0 ** -11 + np.abs(z) * 2.0 ** -11 + 1e-6)
    assert np.all(np.abs(x - xhat) <= 0.5 * s + slack)
    # the extremes land on the ends of the code range
    assert np.all(q[np.arange(512), x.argmin(axis=1)] == 0)
    assert np.all(q[np.arange(512), x.argmax(axis=1)] == 7)


def test_brute_force_nearest_grid_point():
    """q is the grid point nearest to x (ties aside): search over all eight codes."""
    x = _tiles(20, shape=(256, 64))
    q, s16, z16 = quantize_u3_rows(x)
    cand = np.arange(8, dtype=np.float64)
    s = s16.astype(np.float64)[:, None, None]
    z = z16.astype(np.float64)[:, None, None]
    grid = (cand[None, None, :] - z) * s                        # [rows, 1, 8]
    d = np.abs(x.astype(np.float64)[..., None] - grid)
    best = d.argmin(axis=-1)
    dsorted = np.sort(d, axis=-1)
    near_tie = (dsorted[..., 1] - dsorted[..., 0]) < 1e-5 * s[..., 0]
    assert np.all((best == q) | near_tie)
    assert near_tie.mean() < 0.01


def test_dequant_fp32_agrees_with_exact_unless_z_tiny():
    x = _tiles(30, shape=(2048, 128))
    q, s16, z16 = quantize_u3_rows(x)
    exact = dequantize_u3_rows(q, s16, z16)
    f32 = ((q.astype(np.float32) - z16.astype(np.float32)[:, None]) * s16.astype(np.float32)[:, None])
    big_z = np.abs(z16.astype(np.float64)) >= 2.0 ** -8
    assert np.array_equal(f32[big_z].astype(np.float64), exact[big_z])


def test_degenerate_vectors():
    x = np.stack([
        np.full(128, 0.75, np.float32),                      # constant: s = 1 path
        np.linspace(1.0, 2.0, 128, dtype=np.float32),         # all positive
        np.linspace(-3.0, -0.5, 128, dtype=np.float32),       # all negative
        np.zeros(128, np.float32),                            # all zero
    ])
    q, s16, z16 = quantize_u3_rows(x)
    assert s16[0] == 1.0 and s16[3] == 1.0
    xhat = dequantize_u3_rows(q, s16, z16)
    assert np.allclose(xhat[0], 0.75, atol=2 ** -10)
    assert np.all(xhat[3] == 0.0)
    for r in (1, 2):
        assert np.all(np.abs(xhat[r] - x[r]) <= 0.51 * float(s16[r]) + 1e-3)


def test_dropped_zero_point_breaks_the_pins():
    """A plausible mistake (dequantise as q * s, forgetting z) fails the grid bound."""
    x = _tiles(40, shape=(64, 128))
    q, s16, z16 = quantize_u3_rows(x)
    wrong = q.astype(np.float64) * s16.astype(np.float64)[:, None]
    assert np.max(np.abs(wrong - x)) > 1.0

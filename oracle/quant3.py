"""3-bit affine quantisation oracle (test infrastructure only).

Page cited: [3bit] "triton-3bit-kv-cache-kernel" (GitHub README): the title
paragraph (uint3 codes 0..7, on-the-fly affine dequantisation) and section 2,
test 3 (fp16 affine dequant x_hat = (q - z) * s and the requant identity
clamp(round(x_hat / s + z), 0, 7) == q).

The page fixes only the dequantisation identity and fp16 scale/zero.  The rule
for choosing s and z is our reading (the README leaves it open): asymmetric min-max
per (token, kv head) vector with a floating zero point in code units.  All steps
in float32, in this order, with no fused multiply-add:

    lo = min_d x_d,  hi = max_d x_d
    s16 = fp16_RNE((hi - lo) / 7)
    z16 = fp16_RNE(-lo / f32(s16))
    degenerate vectors (s16 zero, subnormal-to-zero or non-finite, or z16
    non-finite): s16 = 1, z16 = fp16_RNE(-lo)
    q_d = clamp(rint(x_d / f32(s16) + f32(z16)), 0, 7)      (rint = half-to-even)

Dequantisation (q - z) * s is evaluated in float64, where it is exact: q - z
needs at most 27 significant bits (q < 8, z an fp16 value whose last bit is no
finer than 2^-24) and its product with an 11-bit s at most 38.  (In float32
it is exact only when z is not tiny; the tests check both facts.)

Pinned by: the section 2 test 3 round trip for every q in 0..7, the grid bound
|x - x_hat| <= s/2 (+ fp16 rounding of s and z), brute-force nearest-grid-point
search, exactness of the dequantisation in fp32 vs fp64, and degenerate vectors.
"""
from __future__ import annotations

import numpy as np


def quantize_u3_rows(x: np.ndarray):
    """x: float32 [..., D] -> (q uint8 [..., D], s16 float16 [...], z16 float16 [...])."""
    x = np.asarray(x, dtype=np.float32)
    lo = np.min(x, axis=-1)
    hi = np.max(x, axis=-1)
    with np.errstate(over="ignore"):          # a range beyond fp16 becomes inf (degenerate)
        s16 = ((hi - lo) / np.float32(7.0)).astype(np.float32).astype(np.float16)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        z16 = ((-lo) / s16.astype(np.float32)).astype(np.float32).astype(np.float16)
    bad = (s16 == 0) | ~np.isfinite(s16) | ~np.isfinite(z16)
    s16 = np.where(bad, np.float16(1.0), s16)
    with np.errstate(over="ignore"):
        z16 = np.where(bad, (-lo).astype(np.float16), z16)
    s = s16.astype(np.float32)[..., None]
    z = z16.astype(np.float32)[..., None]
    with np.errstate(invalid="ignore", over="ignore"):
        t = ((x / s).astype(np.float32) + z).astype(np.float32)
        q = np.clip(np.rint(t), 0, 7).astype(np.uint8)
    return q, s16, z16


def dequantize_u3_rows(q: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """(q - z) * s, exact, as float64 (see module docstring)."""
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)[..., None]
    z = np.asarray(z16, dtype=np.float16).astype(np.float64)[..., None]
    return (np.asarray(q).astype(np.float64) - z) * s

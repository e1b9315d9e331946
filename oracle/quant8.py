"""fp8 e5m2 and int8 cache quantisers (test infrastructure only).

Pages cited: [Append] "Write Triton Kv Cache Append Kernel" (skillsdirectory.com),
  * Inputs the agent should gather first, item 4 (fp8 or int8 caches, fp32 scales) and
    item 8 (the scales' shape and indexing),
  * Required reasoning process, step 6 (divide by the scale in fp32, then cast; fp8 may be
    e4m3 or e5m2),
  * Correctness requirements (the dequantised cache is within one quantisation step).

The e5m2 format is OCP FP8 "E5M2": 1 sign bit, 5 exponent bits with bias 15, 2 mantissa
bits; exponent field 31 holds the infinities (mantissa 0) and NaNs; the largest finite
magnitude is 1.75 * 2^15 = 57344; exponent field 0 holds the subnormals m * 2^-16.  The
table below is written from that definition and the encoder searches it.

Readings of the pages (taken where they leave a step open), by analogy with the e4m3fn cache:
  * one fp32 scale per (block, slot, kv head), computed by the append from its own row:
    s = absmax / 57344 (e5m2) or s = absmax / 127 (int8); s = 1 for an all-zero row;
  * y = x / s in fp32 (correctly rounded);
  * e5m2: y clamped to [-57344, 57344], then the nearest finite e5m2 value, ties to the
    even code, the sign of zero kept;
  * int8: round half to even (np.rint) and clamp to [-127, 127], a symmetric range, so the
    code -128 is never written;
  * inputs are finite.

Pinned by (tests/test_oracle_quant8.py): torch's float8_e5m2 decode of all 256 codes and
its CPU cast over every fp32 value of the clamped range near the format's grid, the
identity of an e5m2 code with the upper byte of the fp16 value it denotes, brute-force
nearest-value search on tiny inputs, int8 ties and saturation worked by hand, and the
one-step round-trip bound for both formats.
"""
from __future__ import annotations

import numpy as np

E5M2_MAX = 57344.0
INT8_MAX = 127


def e5m2_decode_table() -> np.ndarray:
    """All 256 codes -> float64 values (+-inf for 0x7C / 0xFC, NaN for 0x7D-0x7F, 0xFD-0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 2) & 0x1F
        m = code & 0x3
        if e == 0x1F:
            out[code] = sign * np.inf if m == 0 else np.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** -16
        else:
            out[code] = sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)
    return out


_TABLE = e5m2_decode_table()
# the finite non-negative values, in code order 0x00 .. 0x7B (increasing)
_POS_CODES = np.arange(0x7C)
_POS_VALS = _TABLE[:0x7C]


def e5m2_decode(codes: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e5m2_encode_rne(y: np.ndarray) -> np.ndarray:
    """float32 values with |y| <= 57344 -> uint8 e5m2 codes, nearest value, ties to even code.

    The magnitude is located in the sorted table of finite non-negative values; of the two
    neighbours the nearer wins, and on a tie the one with an even code (even mantissa).
    """
    y = np.asarray(y, dtype=np.float32)
    if np.any(np.abs(y) > E5M2_MAX) or not np.all(np.isfinite(y)):
        raise ValueError("e5m2_encode_rne expects finite |y| <= 57344 (clamp first)")
    a = np.abs(y).astype(np.float64)
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    return code | sign


def quantize_e5m2_rows(x: np.ndarray):
    """x: float32 [..., D] -> (codes uint8 [..., D], scale float32 [...]).

    In float32: a = max |x_d|; s = a / 57344 (1 if a == 0); y_d = clamp(x_d / s, +-57344);
    code_d = RNE_e5m2(y_d).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = np.where(a == 0, np.float32(1.0), a / np.float32(E5M2_MAX)).astype(np.float32)
    y = (x / s[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-E5M2_MAX), np.float32(E5M2_MAX))
    return e5m2_encode_rne(y), s


def quantize_int8_rows(x: np.ndarray):
    """x: float32 [..., D] -> (codes int8 [..., D], scale float32 [...]).

    In float32: a = max |x_d|; s = a / 127 (1 if a == 0); code_d = clamp(rint(x_d / s), +-127).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = np.where(a == 0, np.float32(1.0), a / np.float32(INT8_MAX)).astype(np.float32)
    y = (x / s[..., None]).astype(np.float32)
    q = np.clip(np.rint(y), -INT8_MAX, INT8_MAX)
    return q.astype(np.int8), s


def dequantize_e5m2_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes [..., D], scale [...] -> float64 decode(code) * s."""
    return e5m2_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def dequantize_int8_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes (int8, or their uint8 bytes) [..., D], scale [...] -> float64 code * s."""
    c = np.asarray(codes).view(np.int8) if np.asarray(codes).dtype == np.uint8 else np.asarray(codes)
    return c.astype(np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


# ---- caller-given scales ("Write Triton Kv Cache Append Kernel", Inputs items 4 and 8, step 6:
# a per-tensor scale is divided out before the cast; per-token, per-head or per-block scales
# are loaded first).  Reading: the caller owns the scale array; the scale of row
# (block, slot, kv head) is scales[block * sb + slot * ss + head * sh], so that
#   per-tensor        (sb, ss, sh) = (0, 0, 0)
#   per-head          (0, 0, 1)
#   per-block         (1, 0, 0)             one scale per physical block
#   per-block-head    (num_kv_heads, 0, 1)
#   per-token-head    (block_size * num_kv_heads, num_kv_heads, 1)   (the append's own layout)
# Scales are positive and finite; the append reads them and never writes them.

def scale_offsets(blocks: np.ndarray, slots: np.ndarray, heads: np.ndarray, strides) -> np.ndarray:
    """Flat offsets of the scales of rows (block, slot, kv head) (broadcast), int64."""
    sb, ss, sh = (int(v) for v in strides)
    return (np.asarray(blocks, np.int64) * sb + np.asarray(slots, np.int64) * ss +
            np.asarray(heads, np.int64) * sh)


def quantize_given_scale(x: np.ndarray, s: np.ndarray, kind: str) -> np.ndarray:
    """x: float32 [..., D], s: float32 [...] (the caller's scales) -> uint8 codes [..., D].

    In float32: y_d = x_d / s (correctly rounded), clamped to the format's range (+-448 for
    e4m3fn, +-57344 for e5m2, +-127 for int8), then the format's round-to-nearest-even cast.
    """
    from .fp8 import e4m3fn_encode_rne, E4M3_MAX
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    if np.any(~np.isfinite(s)) or np.any(s <= 0):
        raise ValueError("scales must be positive and finite")
    y = (x / s[..., None]).astype(np.float32)
    if kind == "fp8":
        return e4m3fn_encode_rne(np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX)))
    if kind == "e5m2":
        return e5m2_encode_rne(np.clip(y, np.float32(-E5M2_MAX), np.float32(E5M2_MAX)))
    if kind == "i8":
        return np.clip(np.rint(y), -INT8_MAX, INT8_MAX).astype(np.int8).view(np.uint8)
    raise ValueError(kind)

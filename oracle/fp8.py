"""fp8 e4m3fn oracle (test infrastructure only).

Pages cited: [Append] "Write Triton Kv Cache Append Kernel" (skillsdirectory.com),
  * Inputs the agent should gather first, item 4 and item 8 (fp8 cache, fp32 scale,
    per-token / per-head granularity),
  * Required reasoning process, step 6 (divide by the scale in fp32, then cast),
  * Kernel design rules (scale before cast), Correctness requirements (round trip
    within one quantisation step), Common failure modes (quantising before scaling).

The page names Triton's float8e4nv, i.e. the OCP FP8 "E4M3" format: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, no infinities, exponent field 15
with mantissa 7 reserved for NaN, largest finite magnitude 1.75 * 2^8 = 448, and
subnormals m * 2^-9 for exponent field 0.  The format table and the encoder
below are written from that definition.

Readings of the pages (taken where they leave a step open):
  * per-token-per-head scale s = absmax / 448 computed by the append itself over
    its own head_dim vector; s = 1 when the vector is all zero;
  * y = x / s in fp32 (correctly rounded), clamped to [-448, 448], then rounded to
    the nearest e4m3fn value with ties to even mantissa; the sign of zero is kept;
  * inputs are finite (non-finite inputs are outside the contract).

Pinned by: torch's CPU float8_e4m3fn cast over every fp32 bit pattern in the
clamped domain (a library special case), torch's decode of all 256 codes, a
brute-force nearest-value search over the format table, and the one-step
round-trip bound of the append page's correctness requirements.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_BIAS = 7
_MAN_BITS = 3
_MIN_NORMAL_EXP = 1 - _BIAS          # -6


def e4m3fn_decode_table() -> np.ndarray:
    """All 256 codes -> float64 values (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> _MAN_BITS) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** (_MIN_NORMAL_EXP - _MAN_BITS)
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - _BIAS)
    return out


_TABLE = e4m3fn_decode_table()


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_encode_rne(y: np.ndarray) -> np.ndarray:
    """float32 values with |y| <= 448 -> uint8 e4m3fn codes, round to nearest even.

    For a magnitude a > 0 the binade exponent e = floor(log2 a) (exact, via frexp)
    is raised to at least -6 (the subnormal binade shares the quantum of the
    smallest normal binade); the quantum there is 2^(e-3); a / quantum is exact in
    float64, np.rint rounds it half-to-even to an integer m in [0, 16]; m == 16
    carries into the next binade.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.any(np.abs(y) > E4M3_MAX) or not np.all(np.isfinite(y)):
        raise ValueError("e4m3fn_encode_rne expects finite |y| <= 448 (clamp first)")
    sign = (np.signbit(y)).astype(np.uint8) << np.uint8(7)
    a = np.abs(y).astype(np.float64)
    _, fexp = np.frexp(a)                   # a = f * 2^fexp, f in [0.5, 1)
    e = np.maximum(fexp.astype(np.int64) - 1, _MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, e - _MAN_BITS)
    m = np.rint(a / quantum).astype(np.int64)          # 0..16
    carry = m == 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    normal = m >= 8                                     # hidden bit present
    exp_field = np.where(normal, e + _BIAS, 0)
    man_field = np.where(normal, m - 8, m)
    code = (exp_field << _MAN_BITS) | man_field
    code = np.where(a == 0, 0, code).astype(np.uint8)
    return code | sign


def quantize_fp8_rows(x: np.ndarray):
    """x: float32 [..., D] -> (codes uint8 [..., D], scale float32 [...]).

    Steps, all in float32: a = max |x_d|; s = a / 448 (s = 1 if a == 0);
    y_d = x_d / s; y_d = clamp(y_d, -448, 448); code_d = RNE_e4m3fn(y_d).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = np.where(a == 0, np.float32(1.0), a / np.float32(E4M3_MAX)).astype(np.float32)
    y = (x / s[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3fn_encode_rne(y), s


def dequantize_fp8_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes [..., D], scale [...] -> float64 decode(code) * s."""
    return e4m3fn_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]

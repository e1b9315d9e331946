"""3-bit packing oracle (test infrastructure only).

Page cited: [3bit] "triton-3bit-kv-cache-kernel" (GitHub README),
section 1A "24-Bit Octet Layout" and section 1B "96-Bit GPU Coalesced Word Layout".

Definition used (section 1A/1B): a packed 3-bit stream stores value j of a
group at stream bits 3j, 3j+1, 3j+2 (least significant bit first), and the
stream is laid out little-endian: stream bit n is bit (n mod 8) of byte n//8,
and equally bit (n mod 32) of the little-endian uint32 word n//32.  Eight
values fill three bytes exactly, thirty-two values fill three uint32 words
exactly, and the word view is the same memory as four consecutive octets.
Values are masked to their low three bits before packing.

Everything here is written from that definition with Python integers and
numpy shifts; no blocking, no straddle special cases: a value that crosses a
byte or word boundary simply has its bits land in two containers.

Pinned by: the section 1A per-byte bit diagram and the section 1B straddle
lanes (golden fixtures), the exhaustive 2^24 left/right-inverse bijection
(section 2, test 1), and walking-ones/zeros lane isolation with the
uint8[12] == little-endian uint32[3] identity (section 2, test 2).
"""
from __future__ import annotations

import numpy as np


def pack3(values: np.ndarray) -> np.ndarray:
    """values: integer array with n % 8 == 0 elements -> uint8 array of 3n/8 bytes.

    Each consecutive group of 8 values becomes the 24-bit integer sum(v_j << 3j),
    stored as its three little-endian bytes.
    """
    v = np.asarray(values).reshape(-1)
    if v.size % 8:
        raise ValueError("pack3 needs a multiple of 8 values")
    g = (v.astype(np.uint32) & np.uint32(7)).reshape(-1, 8)
    word = np.zeros(g.shape[0], dtype=np.uint32)
    for j in range(8):
        word |= g[:, j] << np.uint32(3 * j)
    out = np.empty((g.shape[0], 3), dtype=np.uint8)
    for byte in range(3):
        out[:, byte] = ((word >> np.uint32(8 * byte)) & np.uint32(0xFF)).astype(np.uint8)
    return out.reshape(-1)


def unpack3(packed: np.ndarray) -> np.ndarray:
    """packed: uint8 array with m % 3 == 0 bytes -> uint8 array of 8m/3 values in 0..7."""
    b = np.asarray(packed, dtype=np.uint8).reshape(-1)
    if b.size % 3:
        raise ValueError("unpack3 needs a multiple of 3 bytes")
    t = b.reshape(-1, 3).astype(np.uint32)
    word = t[:, 0] | (t[:, 1] << np.uint32(8)) | (t[:, 2] << np.uint32(16))
    out = np.empty((t.shape[0], 8), dtype=np.uint8)
    for j in range(8):
        out[:, j] = ((word >> np.uint32(3 * j)) & np.uint32(7)).astype(np.uint8)
    return out.reshape(-1)


def pack3_words(values: np.ndarray) -> np.ndarray:
    """values: n % 32 == 0 integers -> uint32 array of 3n/32 words (section 1B layout).

    Built directly as a 96-bit integer per group of 32 (value i at bit 3i), then
    split into three 32-bit words, word 0 holding the least significant bits.
    """
    v = np.asarray(values).reshape(-1)
    if v.size % 32:
        raise ValueError("pack3_words needs a multiple of 32 values")
    g = v.reshape(-1, 32)
    out = np.empty((g.shape[0], 3), dtype=np.uint32)
    for r in range(g.shape[0]):
        x = 0
        for i in range(32):
            x |= (int(g[r, i]) & 7) << (3 * i)
        for w in range(3):
            out[r, w] = (x >> (32 * w)) & 0xFFFFFFFF
    return out.reshape(-1)


def unpack3_words(words: np.ndarray) -> np.ndarray:
    """words: uint32 array with m % 3 == 0 -> 32m/3 values; value i = bits 3i..3i+2
    of the 96-bit integer W0 + W1*2^32 + W2*2^64."""
    w = np.asarray(words).astype(np.uint64).reshape(-1)
    if w.size % 3:
        raise ValueError("unpack3_words needs a multiple of 3 words")
    t = w.reshape(-1, 3)
    out = np.empty((t.shape[0], 32), dtype=np.uint8)
    for r in range(t.shape[0]):
        x = int(t[r, 0]) | (int(t[r, 1]) << 32) | (int(t[r, 2]) << 64)
        for i in range(32):
            out[r, i] = (x >> (3 * i)) & 7
    return out.reshape(-1)


def pack_rows_u3(q: np.ndarray) -> np.ndarray:
    """q: uint8 codes [..., D] with D % 32 == 0 -> uint32 words [..., 3*D/32].

    Element d of a vector goes to group d // 32, lane d % 32 (ascending d), and
    each group occupies three consecutive words.  Vectorised form of pack3
    (the word view of consecutive octets is the same memory, section 1B)."""
    q = np.asarray(q)
    D = q.shape[-1]
    if D % 32:
        raise ValueError("row length must be a multiple of 32")
    lead = q.shape[:-1]
    octet_bytes = pack3(q.reshape(-1))                      # 3 bytes per 8 values
    return octet_bytes.view("<u4").reshape(*lead, 3 * D // 32)


def unpack_rows_u3(words: np.ndarray, head_dim: int) -> np.ndarray:
    """Inverse of pack_rows_u3: uint32 words [..., 3*D/32] -> uint8 codes [..., D]."""
    words = np.ascontiguousarray(np.asarray(words).astype("<u4"))
    lead = words.shape[:-1]
    if words.shape[-1] * 32 != 3 * head_dim:
        raise ValueError("word count does not match head_dim")
    return unpack3(words.reshape(-1).view(np.uint8)).reshape(*lead, head_dim)

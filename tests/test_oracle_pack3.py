"""Pins of the 3-bit packing oracle against what the 3-bit page fixes.

Page: "triton-3bit-kv-cache-kernel" README, section 1A (octet layout diagram,
straddling values v2 and v5), section 1B (lane i at bit 3i, word (3i)//32, shift
(3i) mod 32; lanes 10 and 21 straddle), section 2 tests 1 and 2 (exhaustive 2^24
bijection both ways; walking-ones/zeros isolation; uint8[12] == LE uint32[3]).
"""
import os

import numpy as np
import pytest

import oracle
from oracle import pack3, unpack3, pack3_words, unpack3_words, pack_rows_u3, unpack_rows_u3


def _read_rows(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---- mutated packers: each is a plausible mistake that some pin must catch -------------
def _pack_msb_first(values):            # bits of each value reversed
    v = np.asarray(values).reshape(-1) & 7
    rev = ((v & 1) << 2) | (v & 2) | ((v >> 2) & 1)
    return pack3(rev)


def _pack_big_endian(values):           # bytes of the 24-bit word in the wrong order
    return pack3(values).reshape(-1, 3)[:, ::-1].reshape(-1)


def _pack_stride4(values):              # values at 4-bit spacing (drops into next octet)
    v = np.asarray(values).reshape(-1, 8).astype(np.uint64) & 7
    word = np.zeros(v.shape[0], dtype=np.uint64)
    for j in range(8):
        word |= v[:, j] << np.uint64(4 * j % 24)
    return np.stack([(word >> np.uint64(8 * k)) & np.uint64(255) for k in range(3)],
                    axis=1).astype(np.uint8).reshape(-1)


def _pack_no_mask(values):              # forgets the & 7 on out-of-range input
    v = np.asarray(values).reshape(-1, 8).astype(np.uint32)
    word = np.zeros(v.shape[0], dtype=np.uint32)
    for j in range(8):
        word |= v[:, j] << np.uint32(3 * j)
    return np.stack([(word >> np.uint32(8 * k)) & np.uint32(255) for k in range(3)],
                    axis=1).astype(np.uint8).reshape(-1)


def layout_pin(pack, golden_dir):
    """Every (value, bit) of the diagram lands on exactly the listed byte bit."""
    for byte, bit, val, vbit in _read_rows(os.path.join(golden_dir, "octet_layout.txt")):
        v = np.zeros(8, dtype=np.uint8)
        v[int(val)] = 1 << int(vbit)
        got = pack(v)
        want = np.zeros(3, dtype=np.uint8)
        want[int(byte)] = 1 << int(bit)
        if not np.array_equal(got, want):
            return False
    return True


def test_octet_layout_matches_diagram(golden_dir):
    assert layout_pin(pack3, golden_dir)


@pytest.mark.parametrize("bad", [_pack_msb_first, _pack_big_endian, _pack_stride4])
def test_layout_pin_catches_mutations(bad, golden_dir):
    assert not layout_pin(bad, golden_dir)


def test_mask_pin_catches_missing_mask():
    v = np.array([0x08, 0xF0, 0, 0, 0, 0, 0, 0x18], dtype=np.uint8)  # only low 3 bits count
    assert np.array_equal(pack3(v), pack3(v & 7))
    assert not np.array_equal(_pack_no_mask(v), pack3(v & 7))


def test_octet_straddles(golden_dir):
    for val, first, last in _read_rows(os.path.join(golden_dir, "octet_straddle.txt")):
        val, first, last = int(val), int(first), int(last)
        v = np.zeros(8, dtype=np.uint8)
        v[val] = 7
        word = int.from_bytes(bytes(pack3(v)), "little")
        assert word == sum(1 << b for b in range(first, last + 1))
        assert first // 8 != last // 8          # really crosses a byte boundary
    # and no other value crosses one
    for val in range(8):
        if val in (2, 5):
            continue
        assert (3 * val) // 8 == (3 * val + 2) // 8


def _bit_home(lane, bit):
    v = np.zeros(32, dtype=np.uint8)
    v[lane] = 1 << bit
    w = pack3_words(v)
    nz = [(i, int(w[i])) for i in range(3) if w[i]]
    assert len(nz) == 1 and bin(nz[0][1]).count("1") == 1
    return nz[0][0], nz[0][1].bit_length() - 1


def test_word96_straddle_lanes(golden_dir):
    rows = _read_rows(os.path.join(golden_dir, "word96_straddle.txt"))
    listed = {}
    for lane, shift, *bits in rows:
        listed[int(lane)] = (int(shift), [tuple(map(int, b.split(":"))) for b in bits])
    straddlers = []
    for lane in range(32):
        homes = [_bit_home(lane, b) for b in range(3)]
        # lane i starts at word (3i)//32, shift (3i) mod 32 (section 1B)
        assert homes[0] == ((3 * lane) // 32, (3 * lane) % 32)
        if len({w for w, _ in homes}) > 1:
            straddlers.append(lane)
            shift, want = listed[lane]
            assert homes == want and homes[0][1] == shift
    assert straddlers == sorted(listed)


def test_hand_derived_vectors(golden_dir):
    for kind, spec, *hexes in _read_rows(os.path.join(golden_dir, "pack3_vectors.txt")):
        n = 8 if kind == "octet" else 32
        v = np.zeros(n, dtype=np.uint8)
        for item in spec.split(","):
            i, val = item.split(":")
            v[int(i)] = int(val)
        if kind == "octet":
            assert list(pack3(v)) == [int(h, 16) for h in hexes]
            assert np.array_equal(unpack3(pack3(v)), v)
        else:
            assert [int(x) for x in pack3_words(v)] == [int(h, 16) for h in hexes]
            assert np.array_equal(unpack3_words(pack3_words(v)), v)


CHUNK = 1 << 21


def test_exhaustive_bijection_2pow24():
    """Section 2 test 1: every v in {0..7}^8 and every b in {0..255}^3."""
    for start in range(0, 1 << 24, CHUNK):
        i = np.arange(start, start + CHUNK, dtype=np.uint32)
        # all octets of values, enumerated as the base-8 digits of i
        digits = np.stack([(i // (8 ** j)) % 8 for j in range(8)], axis=1).astype(np.uint8)
        le_bytes = np.stack([(i >> np.uint32(8 * k)) & np.uint32(255) for k in range(3)],
                            axis=1).astype(np.uint8)
        packed = pack3(digits)
        # closed form: packing the base-8 digits of i gives the little-endian bytes of i
        assert np.array_equal(packed, le_bytes.reshape(-1))
        # left inverse
        assert np.array_equal(unpack3(packed), digits.reshape(-1))
        # right inverse, over all byte triples (le_bytes enumerates {0..255}^3)
        assert np.array_equal(pack3(unpack3(le_bytes.reshape(-1))), le_bytes.reshape(-1))


@pytest.mark.parametrize("background", [0, 7])
def test_walking_pattern_isolation(background):
    """Section 2 test 2: all 32 lanes x 8 values over both backgrounds; zero
    bit-bleed outside the lane's three bits; uint8[12] equals LE uint32[3]."""
    base = np.full(32, background, dtype=np.uint8)
    base_words = pack3_words(base)
    base_int = sum(int(base_words[w]) << (32 * w) for w in range(3))
    for lane in range(32):
        for val in range(8):
            v = base.copy()
            v[lane] = val
            words = pack3_words(v)
            octets = pack3(v)                                   # 12 bytes
            assert np.array_equal(octets.view("<u4"), words)    # LE equivalence
            assert np.array_equal(unpack3_words(words), v)
            assert np.array_equal(unpack3(octets), v)
            x = sum(int(words[w]) << (32 * w) for w in range(3))
            diff = x ^ base_int
            assert diff & ~(7 << (3 * lane)) == 0                # no bleed into other lanes


def test_rows_form_matches_group_form():
    rng = np.random.default_rng(7)
    q = rng.integers(0, 8, size=(5, 3, 128), dtype=np.uint8)
    words = pack_rows_u3(q)
    assert words.shape == (5, 3, 12)
    for idx in np.ndindex(5, 3):
        assert np.array_equal(words[idx], pack3_words(q[idx]))
    assert np.array_equal(unpack_rows_u3(words, 128), q)
    q64 = rng.integers(0, 8, size=(4, 64), dtype=np.uint8)
    assert np.array_equal(unpack_rows_u3(pack_rows_u3(q64), 64), q64)


def test_oracle_header_declares_test_infrastructure():
    assert "TEST INFRASTRUCTURE ONLY" in oracle.__doc__

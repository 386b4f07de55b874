"""Pins for the oracle's Q4_K decode (CPU only).

The pages name the format (muser-book ch. 8, section 8.2); the layout is the
GGUF one. Pins: numpy's independent fp16 conversion, hand-derived bytes,
a round trip through the independent test-side packer, and exact rational
arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.q4k_pack import f16_bits, pack_block, pack_quants, pack_scales_mins


def test_half_to_double_matches_numpy_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b in range(0, 65536, 1):
        r = ref[b]
        got = oracle.half_to_double(b)
        if np.isfinite(r):
            assert got == r or (got == 0 and r == 0), b
            assert np.signbit(got) == np.signbit(r), b
        else:
            assert np.isnan(got), b


def test_scale_bytes_hand_derived():
    # Twelve bytes with every 6-bit field decoded by hand from the layout:
    # sc[0..3]/m[0..3] are the low six bits of bytes 0..3/4..7; sc[4..7] and
    # m[4..7] take their low four bits from the low/high nibble of bytes
    # 8..11 and their top two bits from the top bits of bytes 0..3/4..7.
    s12 = bytes([0xC1, 0x3F, 0x85, 0x40, 0x7F, 0x00, 0xE1, 0x0A, 0x5F, 0x12, 0xA0, 0x07])
    sc, mn = oracle.scales_mins(s12)
    assert list(sc) == [1, 63, 5, 0, 63, 2, 32, 23]
    assert list(mn) == [63, 0, 33, 10, 21, 1, 58, 0]


def test_scale_pack_unpack_round_trip_is_bijection():
    g = np.random.default_rng(7)
    for _ in range(2000):
        s12 = bytes(g.integers(0, 256, 12, dtype=np.uint8))
        sc, mn = oracle.scales_mins(s12)
        assert all(0 <= v < 64 for v in list(sc) + list(mn))
        assert pack_scales_mins(sc, mn) == s12
    # and the other direction: chosen fields survive pack -> decode
    for _ in range(2000):
        sc = g.integers(0, 64, 8)
        mn = g.integers(0, 64, 8)
        got_sc, got_mn = oracle.scales_mins(pack_scales_mins(sc, mn))
        assert list(got_sc) == list(sc) and list(got_mn) == list(mn)


def test_quant_layout_hand_derived():
    # Q byte i holds value i: low nibble i & 15, high nibble i >> 4.
    # d = 1, dmin = 0, every scale 1 -> weights are the raw nibbles.
    blk = bytes([0x00, 0x3C, 0x00, 0x00]) + pack_scales_mins([1] * 8, [0] * 8) + bytes(range(128))
    w = oracle.decode_block(blk)
    expect = {0: 0, 1: 1, 15: 15, 16: 0, 31: 15,       # group 0 low nibbles of bytes 0..31
              32: 0, 47: 0, 48: 1, 63: 1,             # group 0 high nibbles of bytes 0..31
              64: 0, 95: 15, 96: 2, 127: 3,           # group 1: bytes 32..63
              128: 0, 160: 4, 191: 5,                 # group 2: bytes 64..95
              192: 0, 223: 15, 224: 6, 255: 7}        # group 3: bytes 96..127
    for i, v in expect.items():
        assert w[i] == v, (i, w[i], v)


def test_hand_block_scales_and_ramp():
    sc = [63, 1, 32, 17, 48, 33, 16, 62]
    mn = [0, 63, 5, 40, 47, 18, 31, 60]
    q = [i % 16 for i in range(256)]
    # d = 1.0 (0x3C00), dmin = 0: w = sc_j * q
    w = oracle.decode_block(pack_block(0x3C00, 0x0000, sc, mn, q))
    for i in range(256):
        assert w[i] == sc[i // 32] * q[i]
    # d = 0, dmin = 1.0: w = -m_j
    w = oracle.decode_block(pack_block(0x0000, 0x3C00, sc, mn, q))
    for i in range(256):
        assert w[i] == -mn[i // 32]
    # d = 0.5 (0x3800), dmin = 2.0 (0x4000)
    w = oracle.decode_block(pack_block(0x3800, 0x4000, sc, mn, q))
    for i in range(256):
        assert w[i] == 0.5 * sc[i // 32] * q[i] - 2.0 * mn[i // 32]


def test_header_is_little_endian():
    # d = 0x3C01 (1 + 2^-10): byte 0 = 0x01, byte 1 = 0x3C
    q = [1] * 256
    w = oracle.decode_block(pack_block(0x3C01, 0, [1] * 8, [0] * 8, q))
    assert w[0] == 1.0 + 2.0 ** -10
    raw = bytes(pack_block(0x3C01, 0, [1] * 8, [0] * 8, q))
    assert raw[0] == 0x01 and raw[1] == 0x3C


def test_decode_exact_against_fractions():
    g = np.random.default_rng(11)
    for _ in range(50):
        d = float(np.float16(g.uniform(0.001, 0.05)))
        dmin = float(np.float16(g.uniform(0.001, 0.05)))
        sc = g.integers(0, 64, 8)
        mn = g.integers(0, 64, 8)
        q = g.integers(0, 16, 256)
        w = oracle.decode_block(pack_block(f16_bits(d), f16_bits(dmin), sc, mn, q))
        for i in range(256):
            exact = Fraction(d) * int(sc[i // 32]) * int(q[i]) - Fraction(dmin) * int(mn[i // 32])
            assert Fraction(w[i]) == exact


def test_nonfinite_header_rejected():
    blk = pack_block(0x7C00, 0, [1] * 8, [0] * 8, [0] * 256)  # d = +inf
    with pytest.raises(ValueError):
        oracle.decode_block(blk)


def test_pack_quants_matches_layout_statement():
    q = list(range(16)) * 16
    b = pack_quants(q)
    assert b[0] == (q[0] | (q[32] << 4))
    assert b[127] == (q[255 - 32] | (q[255] << 4))

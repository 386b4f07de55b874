"""Pins for the oracle's Q5_K and Q6_K decode and their products (CPU only).

The pages say the draft loads Q4_K, Q5_K and Q6_K tensors and that its v
projection is Q6_K (muser-book ch. 8, section 8.2); the byte layouts are the
GGUF ones. Pins: weights worked out by hand from the layout statement, a
round trip through the independent test-side packers, exact rational
arithmetic, and closed forms of the product.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic
from tests.q4k_pack import f16_bits, pack_q5k_block, pack_q6k_block, pack_scales_mins

ONE = 0x3C00  # fp16 1.0


# ------------------------------------------------------------------- Q5_K

def test_q5k_quant_layout_hand_derived():
    # nibble byte b = b; fifth-bit byte l = 1 << (l % 8); d = 1, dmin = 0,
    # every scale 1, so each weight is its 5-bit quant. Worked by hand:
    # weight i: nibble byte 32 (i // 64) + i % 32 (low nibble when i % 64 <
    # 32), fifth bit = bit i // 32 of byte i % 32.
    qh = bytes([1 << (l % 8) for l in range(32)])
    blk = bytes([0x00, 0x3C, 0x00, 0x00]) + pack_scales_mins([1] * 8, [0] * 8) + qh + bytes(range(128))
    w = oracle.decode_block(blk, "q5k")
    expect = {0: 16, 1: 1, 33: 16, 66: 18, 99: 18, 100: 2, 224: 6, 231: 22, 255: 23}
    for i, v in expect.items():
        assert w[i] == v, (i, w[i], v)


def test_q5k_scales_mins_and_header():
    sc = [63, 1, 32, 17, 48, 33, 16, 62]
    mn = [0, 63, 5, 40, 47, 18, 31, 60]
    q = [(7 * i) % 32 for i in range(256)]
    w = oracle.decode_block(pack_q5k_block(ONE, 0, sc, mn, q), "q5k")
    assert all(w[i] == sc[i // 32] * q[i] for i in range(256))
    w = oracle.decode_block(pack_q5k_block(0, ONE, sc, mn, q), "q5k")
    assert all(w[i] == -mn[i // 32] for i in range(256))
    # d = 1 + 2^-10 stored little-endian
    raw = pack_q5k_block(0x3C01, 0, [1] * 8, [0] * 8, [1] * 256)
    assert raw[0] == 0x01 and raw[1] == 0x3C
    assert oracle.decode_block(raw, "q5k")[0] == 1.0 + 2.0 ** -10


def test_q5k_round_trip_and_exact_decode():
    g = np.random.default_rng(21)
    lib = oracle._load()
    for _ in range(300):
        raw = bytes(g.integers(0, 256, 176, dtype=np.uint8))
        b = np.frombuffer(raw, dtype=np.uint8).copy()
        q = [lib.kqo_quant_q5k(oracle._p(b[16:]), oracle._p(b[48:]), i) for i in range(256)]
        sc, mn = oracle.scales_mins(raw[4:16])
        assert pack_q5k_block(raw[0] | raw[1] << 8, raw[2] | raw[3] << 8, sc, mn, q) == raw
    for _ in range(40):
        d = float(np.float16(g.uniform(0.001, 0.05)))
        dmin = float(np.float16(g.uniform(0.001, 0.05)))
        sc, mn, q = g.integers(0, 64, 8), g.integers(0, 64, 8), g.integers(0, 32, 256)
        w = oracle.decode_block(pack_q5k_block(f16_bits(d), f16_bits(dmin), sc, mn, q), "q5k")
        for i in range(256):
            assert Fraction(w[i]) == Fraction(d) * int(sc[i // 32]) * int(q[i]) - Fraction(dmin) * int(mn[i // 32])


# ------------------------------------------------------------------- Q6_K

def test_q6k_quant_layout_hand_derived():
    # nibble byte b = b, high-part byte b = b, scales all 1, d = 1 at the
    # end: each weight is q - 32. Worked by hand from the layout (weight i of
    # half h, quarter c, lane l: nibble byte 64 h + l + 32 (c & 1), low for
    # c < 2; top bits 2c..2c+1 of high-part byte 32 h + l).
    blk = bytes(range(128)) + bytes(range(64)) + bytes([1] * 16) + bytes([0x00, 0x3C])
    w = oracle.decode_block(blk, "q6k")
    expect = {0: -32, 1: -15, 33: -31, 66: -32, 127: -29, 128: -32, 140: -20, 175: 31, 200: 4, 255: -25}
    for i, v in expect.items():
        assert w[i] == v, (i, w[i], v)


def test_q6k_signed_scales_and_header():
    scales = [-128, 127, -1, 0, 1, 2, -64, 63, 5, -5, 100, -100, 17, -17, 32, -32]
    q = [(5 * i + 3) % 64 for i in range(256)]
    w = oracle.decode_block(pack_q6k_block(ONE, scales, q), "q6k")
    assert all(w[i] == scales[i // 16] * (q[i] - 32) for i in range(256))
    # scale byte 0x80 is -128 (two's complement)
    raw = pack_q6k_block(ONE, scales, q)
    assert raw[192] == 0x80 and raw[193] == 0x7F
    # d is the last two bytes, little-endian
    raw = pack_q6k_block(0x3C01, [1] * 16, [33] * 256)
    assert raw[208] == 0x01 and raw[209] == 0x3C
    assert oracle.decode_block(raw, "q6k")[0] == 1.0 + 2.0 ** -10
    # extremes: q = 0 and 63 with scale -128 give 4,096 and -4,031
    w = oracle.decode_block(pack_q6k_block(ONE, [-128] * 16, [0] * 128 + [63] * 128), "q6k")
    assert w[0] == 4096 and w[255] == -128 * 31


def test_q6k_round_trip_and_exact_decode():
    g = np.random.default_rng(22)
    lib = oracle._load()
    for _ in range(300):
        raw = bytes(g.integers(0, 256, 210, dtype=np.uint8))
        b = np.frombuffer(raw, dtype=np.uint8).copy()
        q = [lib.kqo_quant_q6k(oracle._p(b), oracle._p(b[128:]), i) for i in range(256)]
        scales = np.frombuffer(raw[192:208], dtype=np.int8)
        assert pack_q6k_block(raw[208] | raw[209] << 8, scales, q) == raw
    for _ in range(40):
        d = float(np.float16(g.uniform(0.0002, 0.01)))
        scales, q = g.integers(-128, 128, 16), g.integers(0, 64, 256)
        w = oracle.decode_block(pack_q6k_block(f16_bits(d), scales, q), "q6k")
        for i in range(256):
            assert Fraction(w[i]) == Fraction(d) * int(scales[i // 16]) * (int(q[i]) - 32)


def test_nonfinite_block_scale_rejected():
    with pytest.raises(ValueError):
        oracle.decode_block(pack_q6k_block(0x7C00, [1] * 16, [0] * 256), "q6k")
    with pytest.raises(ValueError):
        oracle.decode_block(pack_q5k_block(0, 0x7E00, [1] * 8, [0] * 8, [0] * 256), "q5k")


# ------------------------------------------------ products of both formats

@pytest.mark.parametrize("fmt", ["q5k", "q6k"])
def test_gemv_exact_rational_brute_force(fmt):
    """Small shapes against Fractions: |L - exact| <= K 2^-53 A."""
    g = np.random.default_rng(23)
    n, k, m = 3, 512, 2
    w = synthetic.kquant_matrix(fmt, n, k, 31)
    x = g.standard_normal((m, k)).astype(np.float32)
    L, A = oracle.gemv_rows(w, k, x, fmt=fmt)
    nb = oracle.block_bytes(fmt)
    for r in range(n):
        wr = np.concatenate([oracle.decode_block(w[r, b * nb:(b + 1) * nb].tobytes(), fmt) for b in range(k // 256)])
        for mm in range(m):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(wr, x[mm]))
            assert abs(Fraction(L[mm, r]) - exact) <= Fraction(k) * Fraction(2.0 ** -53) * Fraction(A[mm, r])


@pytest.mark.parametrize("fmt", ["q5k", "q6k"])
def test_gemv_one_hot_rows_extract_weight_columns(fmt):
    n, k = 5, 512
    w = synthetic.kquant_matrix(fmt, n, k, 41)
    cols = [0, 1, 31, 32, 100, 255, 256, 300, 511]
    x = np.zeros((len(cols), k), np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    L, _ = oracle.gemv_rows(w, k, x, fmt=fmt)
    W = oracle.decode_matrix(w, k, fmt)
    for i, c in enumerate(cols):
        assert np.array_equal(L[i], W[:, c])


def test_q6k_all_offsets_closed_form():
    """q = 32 everywhere makes every weight 0; q = 0 with x = 1 gives
    L = -32 d sum of scales (one block)."""
    scales = list(range(-8, 8))
    x = np.ones((1, 256), np.float32)
    w0 = np.frombuffer(pack_q6k_block(ONE, scales, [32] * 256), np.uint8)[None, :]
    L, A = oracle.gemv_rows(w0, 256, x, fmt="q6k")
    assert L[0, 0] == 0 and A[0, 0] == 0
    w1 = np.frombuffer(pack_q6k_block(0x3800, scales, [0] * 256), np.uint8)[None, :]  # d = 0.5
    L, _ = oracle.gemv_rows(w1, 256, x, fmt="q6k")
    assert L[0, 0] == -32 * 0.5 * 16 * sum(scales)


def test_q5k_fifth_bit_closed_form():
    """Only the fifth bits set (nibbles 0), d = 1, sc = 1, dmin = 0, x = 1:
    L = 16 x (number of set fifth bits)."""
    g = np.random.default_rng(24)
    q = [16 * int(b) for b in g.integers(0, 2, 256)]
    w = np.frombuffer(pack_q5k_block(ONE, 0, [1] * 8, [0] * 8, q), np.uint8)[None, :]
    L, _ = oracle.gemv_rows(w, 256, np.ones((1, 256), np.float32), fmt="q5k")
    assert L[0, 0] == sum(q)


def test_synthetic_q56_fields():
    w5 = synthetic.q5k_matrix(64, 512, 3)
    assert w5.shape == (64, 2 * 176)
    d = w5.reshape(-1, 176)[:, 0:4].copy().view(np.float16).astype(np.float64)
    assert d.min() >= 0.001 - 1e-6 and d.max() <= 0.05 + 1e-4
    w6 = synthetic.q6k_matrix(64, 512, 3)
    assert w6.shape == (64, 2 * 210)
    d6 = w6.reshape(-1, 210)[:, 208:210].copy().view(np.float16).astype(np.float64)
    assert d6.min() >= 0.0002 - 1e-6 and d6.max() <= 0.01 + 1e-5
    assert np.array_equal(w6, synthetic.q6k_matrix(64, 512, 3))
    sc = w6.reshape(-1, 210)[:, 192:208].view(np.int8)
    assert sc.min() == -128 and sc.max() == 127

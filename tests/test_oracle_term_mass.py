"""Pins for the oracle's term mass B = sum_k (|d sc_j q_k| + |dmin m_j|) |x_k|
(CPU only): the quantity a kernel that forms a block's scale term and min term
apart has its rounding error proportional to.

Each pin fixes B by other means than the oracle's own formula: B equals the
tolerance mass A exactly when either term vanishes (dmin = 0, or every quant
0); on a hand-built block whose two terms cancel for every weight (so w = 0
and A = 0) B has a closed form; and B >= A holds on random matrices, with
the excess over A equal to twice the mass of the cancelled part on a block
built so that exactly one sub-block mixes both terms.
"""
import numpy as np

import oracle
import synthetic
from tests.q4k_pack import f16_bits, pack_block, pack_matrix


def _rand_fields(rng):
    sc = [int(v) for v in rng.integers(0, 64, 8)]
    mn = [int(v) for v in rng.integers(0, 64, 8)]
    q = [int(v) for v in rng.integers(0, 16, 256)]
    return sc, mn, q


def test_equals_tolerance_mass_when_min_term_is_zero():
    rng = np.random.default_rng(11)
    blocks = []
    for r in range(6):
        row = []
        for b in range(2):
            sc, mn, q = _rand_fields(rng)
            d = float(rng.uniform(0.001, 0.05))
            row.append(pack_block(f16_bits(d), f16_bits(0.0), sc, mn, q))
        blocks.append(row)
    w = pack_matrix(blocks)
    x = synthetic.activations(3, 512, 12)
    L, A = oracle.gemv_rows(w, 512, x)
    B = oracle.term_mass(w, 512, x)
    assert np.array_equal(A, B)


def test_equals_tolerance_mass_when_quants_are_zero():
    rng = np.random.default_rng(13)
    blocks = []
    for r in range(5):
        sc, mn, _ = _rand_fields(rng)
        dmin = float(rng.uniform(0.001, 0.05))
        blocks.append([pack_block(f16_bits(0.03), f16_bits(dmin), sc, mn, [0] * 256)])
    w = pack_matrix(blocks)
    x = synthetic.activations(2, 256, 14)
    _, A = oracle.gemv_rows(w, 256, x)
    B = oracle.term_mass(w, 256, x)
    assert np.array_equal(A, B)


def test_cancelling_block_closed_form():
    """d = dmin = 2^-6, every scale 4, every quant 15, every min 60: each
    weight is 2^-6 (4 * 15 - 60) = 0, so L = A = 0, while B = 2 * 2^-6 * 60 *
    sum |x| exactly (all values dyadic with short significands)."""
    d = f16_bits(2.0 ** -6)
    blk = pack_block(d, d, [4] * 8, [60] * 8, [15] * 256)
    w = pack_matrix([[blk]])
    x = np.arange(-128, 128, dtype=np.float32)[None, :] * np.float32(0.25)
    L, A = oracle.gemv_rows(w, 256, x)
    B = oracle.term_mass(w, 256, x)
    assert L[0, 0] == 0.0 and A[0, 0] == 0.0
    assert B[0, 0] == 2 * 2.0 ** -6 * 60 * float(np.abs(x).astype(np.float64).sum())


def test_one_mixed_sub_block_adds_twice_its_cancelled_mass():
    """Sub-block 3 alone has both terms (sc = 2, q = 5 or 9, m = 4, d = dmin
    = 1/8): its weights are 1/8 (2 q - 4) > 0, and B - A there is twice
    dmin * m * |x| summed over the sub-block. Everywhere else m = 0."""
    d = f16_bits(0.125)
    sc = [1, 3, 2, 2, 5, 1, 7, 4]
    mn = [0, 0, 0, 4, 0, 0, 0, 0]
    q = [(i * 7) % 16 for i in range(256)]
    for i in range(96, 128):
        q[i] = 5 if i % 2 else 9
    w = pack_matrix([[pack_block(d, d, sc, mn, q)]])
    x = synthetic.activations(2, 256, 15)
    _, A = oracle.gemv_rows(w, 256, x)
    B = oracle.term_mass(w, 256, x)
    for r in range(2):
        expect = 2 * 0.125 * 4 * float(np.abs(x[r, 96:128]).astype(np.float64).sum())
        assert abs((B[r, 0] - A[r, 0]) - expect) <= 1e-12 * B[r, 0]


def test_not_below_tolerance_mass_and_rows_subset():
    w = synthetic.q4k_matrix(20, 1024, 16)
    x = synthetic.activations(4, 1024, 17)
    _, A = oracle.gemv_rows(w, 1024, x)
    B = oracle.term_mass(w, 1024, x)
    assert np.all(B >= A)
    rows = [19, 0, 7]
    assert np.array_equal(oracle.term_mass(w, 1024, x, rows=rows), B[:, rows])

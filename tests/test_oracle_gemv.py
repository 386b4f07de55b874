"""Pins for the oracle's logits L = W x^T and tolerance mass A (CPU only).

Exact rational brute force on tiny shapes, closed forms for one-hot and
constant activations and for zero quants, the integer-dot special case, and
row invariance (row i of an M-row call equals an M=1 call).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic
from tests.q4k_pack import f16_bits, pack_block, pack_matrix


def _exact_weights(w_bytes: np.ndarray, k: int):
    """Exact weights as Fractions, decoded here from the field definitions
    (d, dmin fp16 via numpy; fields via the layout statement)."""
    n = w_bytes.shape[0]
    out = []
    for r in range(n):
        row = []
        for b in range(k // 256):
            blk = bytes(w_bytes[r, b * 144:(b + 1) * 144])
            d = Fraction(float(np.frombuffer(blk[0:2], dtype=np.float16)[0]))
            dm = Fraction(float(np.frombuffer(blk[2:4], dtype=np.float16)[0]))
            s = blk[4:16]
            sc = [s[j] & 63 for j in range(4)] + [(s[j + 8] & 15) | ((s[j] >> 6) << 4) for j in range(4)]
            mn = [s[j + 4] & 63 for j in range(4)] + [(s[j + 8] >> 4) | ((s[j + 4] >> 6) << 4) for j in range(4)]
            qb = blk[16:]
            for i in range(256):
                g, l = divmod(i, 64)
                byte = qb[32 * g + (l % 32)]
                q = (byte & 15) if l < 32 else (byte >> 4)
                row.append(d * sc[i // 32] * q - dm * mn[i // 32])
        out.append(row)
    return out


@pytest.mark.parametrize("n,k,m", [(3, 256, 1), (8, 256, 4), (5, 512, 3), (2, 512, 2)])
def test_exact_rational_brute_force(n, k, m):
    w = synthetic.q4k_matrix(n, k, seed=100 + n + k + m)
    x = synthetic.activations(m, k, seed=200 + n + k + m)
    L, A = oracle.gemv_rows(w, k, x)
    W = _exact_weights(w, k)
    for mm in range(m):
        xs = [Fraction(float(v)) for v in x[mm]]
        for r in range(n):
            exact = sum(W[r][kk] * xs[kk] for kk in range(k))
            mass = sum(abs(W[r][kk] * xs[kk]) for kk in range(k))
            bound = (k + 1) * 2.0 ** -53 * float(mass)
            assert abs(Fraction(L[mm, r]) - exact) <= Fraction(bound)
            assert abs(Fraction(A[mm, r]) - mass) <= Fraction(bound)


def test_one_hot_rows_extract_weight_columns():
    n, k = 40, 1024
    w = synthetic.q4k_matrix(n, k, seed=5)
    Wd = oracle.decode_matrix(w, k)
    cols = [0, 1, 255, 256, 511, 777, 1023]
    x = np.zeros((len(cols), k), dtype=np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    L, A = oracle.gemv_rows(w, k, x)
    for i, c in enumerate(cols):
        assert np.array_equal(L[i], Wd[:, c])
        assert np.array_equal(A[i], np.abs(Wd[:, c]))


def _rand_fields(g):
    d = float(np.float16(g.uniform(0.001, 0.05)))
    dm = float(np.float16(g.uniform(0.001, 0.05)))
    return d, dm, g.integers(0, 64, 8), g.integers(0, 64, 8)


def test_zero_quants_give_minus_min_term():
    g = np.random.default_rng(3)
    k, n = 512, 6
    rows, dms, mns = [], [], []
    for r in range(n):
        blocks = []
        for b in range(k // 256):
            d, dm, sc, mn = _rand_fields(g)
            blocks.append(pack_block(f16_bits(d), f16_bits(dm), sc, mn, [0] * 256))
            dms.append(dm); mns.append(mn)
        rows.append(blocks)
    w = pack_matrix(rows)
    x = synthetic.activations(2, k, seed=9)
    L, _ = oracle.gemv_rows(w, k, x)
    for r in range(n):
        for mm in range(2):
            expect = 0.0
            for b in range(k // 256):
                dm, mn = dms[r * (k // 256) + b], mns[r * (k // 256) + b]
                for j in range(8):
                    s = np.sum(x[mm, b * 256 + 32 * j: b * 256 + 32 * j + 32].astype(np.float64))
                    expect -= dm * mn[j] * s
            assert L[mm, r] == pytest.approx(expect, rel=1e-12, abs=1e-12)


def test_constant_activation_closed_form():
    g = np.random.default_rng(4)
    k, n = 768, 5
    rows, info = [], []
    for r in range(n):
        blocks = []
        for b in range(k // 256):
            d, dm, sc, mn = _rand_fields(g)
            q = g.integers(0, 16, 256)
            blocks.append(pack_block(f16_bits(d), f16_bits(dm), sc, mn, q))
            info.append((d, dm, sc, mn, q))
        rows.append(blocks)
    w = pack_matrix(rows)
    x = np.ones((1, k), dtype=np.float32)
    L, A = oracle.gemv_rows(w, k, x)
    for r in range(n):
        expect = Fraction(0)
        for b in range(k // 256):
            d, dm, sc, mn, q = info[r * (k // 256) + b]
            for j in range(8):
                expect += Fraction(d) * int(sc[j]) * int(np.sum(q[32 * j:32 * j + 32])) - 32 * Fraction(dm) * int(mn[j])
        assert L[0, r] == float(expect)  # every partial sum is exact here


def test_integer_dot_special_case():
    g = np.random.default_rng(6)
    k, n = 1024, 7
    qs, rows = [], []
    for r in range(n):
        blocks = []
        for b in range(k // 256):
            q = g.integers(0, 16, 256)
            qs.append(q)
            blocks.append(pack_block(0x3C00, 0x0000, [1] * 8, [0] * 8, q))
        rows.append(blocks)
    w = pack_matrix(rows)
    xi = g.integers(-50, 51, size=(3, k))
    L, _ = oracle.gemv_rows(w, k, xi.astype(np.float32))
    Q = np.stack([np.concatenate(qs[r * 4:(r + 1) * 4]) for r in range(n)])
    assert np.array_equal(L, (xi @ Q.T).astype(np.float64))


def test_row_invariance_and_row_subset():
    n, k, m = 64, 2048, 16
    w = synthetic.q4k_matrix(n, k, seed=12)
    x = synthetic.activations(m, k, seed=13)
    L, A = oracle.gemv_rows(w, k, x)
    for i in [0, 5, 15]:
        L1, A1 = oracle.gemv_rows(w, k, x[i:i + 1])
        assert np.array_equal(L1[0], L[i]) and np.array_equal(A1[0], A[i])
    rows = [63, 0, 17, 17, 40]
    Ls, As = oracle.gemv_rows(w, k, x, rows=rows)
    assert np.array_equal(Ls, L[:, rows]) and np.array_equal(As, A[:, rows])


def test_threads_do_not_change_results():
    n, k, m = 96, 1024, 4
    w = synthetic.q4k_matrix(n, k, seed=14)
    x = synthetic.activations(m, k, seed=15)
    L1, A1 = oracle.gemv_rows(w, k, x, threads=1)
    L8, A8 = oracle.gemv_rows(w, k, x, threads=8)
    assert np.array_equal(L1, L8) and np.array_equal(A1, A8)


def test_rejects_bad_inputs():
    w = synthetic.q4k_matrix(4, 256, seed=1)
    x = synthetic.activations(1, 256, seed=1)
    x[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.gemv_rows(w, 256, x)
    with pytest.raises(ValueError):
        oracle.gemv_rows(w, 512, synthetic.activations(1, 512, seed=1))

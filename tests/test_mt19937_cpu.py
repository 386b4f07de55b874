"""The library's pinned draw stream (kq_mt19937_*) and the decision that
consumes it (kq_speculative_decide_mt), on the host (no GPU needed).

* Words: the value the C++ standard fixes for std::mt19937 (the 10,000th
  output after seeding 5489 is 4,123,659,995) and numpy's MT19937 with the
  reference-code (legacy) seeding, word for word, for several seeds and
  split into calls of awkward sizes (state regenerations inside a call).
* Float draws: equal to the oracle's conversion of the same words.
* The decision: bit for bit the oracle's speculative_decide_mt from the
  same seed, and the two generators in the same state afterwards (the
  library's next word equals the oracle's next word).
* Errors: nothing drawn and nothing written on any refused call.
"""
import ctypes

import numpy as np
import pytest

from oracle.mt19937 import MT19937 as OracleMT
from oracle.mt19937 import to_uniform_f32
from oracle.stochastic import speculative_decide_mt as oracle_decide_mt
from quant_verify_gemv_amd import lib as kq

NULL, SHAPE, TOKEN = 1, 2, 4


def test_tenthousandth_output_of_default_seed():
    g = kq.MT19937()
    assert int(g.u32(10000)[-1]) == 4123659995


@pytest.mark.parametrize("seed", [0, 1, 5489, 0x9E3779B9, 2 ** 32 - 1])
def test_words_match_numpy_reference_seeding(seed):
    bg = np.random.MT19937()
    bg._legacy_seeding(seed)
    want = bg.random_raw(3 * 624 + 100)
    g = kq.MT19937(seed)
    got, done = [], 0
    for size in (1, 623, 2, 624, 0, 700, 1000):
        size = min(size, len(want) - done)
        got.append(g.u32(size))
        done += size
    assert np.array_equal(np.concatenate(got).astype(np.uint64), want[:done])


def test_float_draws_match_oracle_conversion():
    g = kq.MT19937(2024)
    words = kq.MT19937(2024).u32(1500)
    u = g.uniform_f32(1500)
    assert u.dtype == np.float32
    assert np.array_equal(u, np.array([to_uniform_f32(w) for w in words], dtype=np.float32))
    assert float(u.min()) >= 0.0 and float(u.max()) < 1.0


def random_case(rng, n, k):
    z = rng.normal(size=(k + 1, n)) * rng.choice([1.0, 4.0])
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    y = rng.normal(size=(k, n)) * rng.choice([1.0, 4.0])
    q = np.exp(y - y.max(axis=1, keepdims=True))
    q = (q / q.sum(axis=1, keepdims=True)).astype(np.float32)
    draft = [int(rng.choice(n, p=q[i] / q[i].sum())) for i in range(k)]
    orders = np.stack([rng.permutation(n) for _ in range(k + 1)]).astype(np.int32)
    return draft, q, p, orders


@pytest.mark.parametrize("n,k", [(5, 3), (64, 7), (300, 15), (9, 0)])
def test_decide_mt_matches_oracle_and_leaves_the_same_state(n, k):
    rng = np.random.default_rng(1000 + n + k)
    outcomes = set()
    for trial in range(150):
        draft, q, p, orders = random_case(rng, n, k)
        if trial % 3 == 0:
            q = p[:k].copy()  # a draft equal to the target: every proposal accepted
        seed = int(rng.integers(0, 2 ** 32))
        g, o = kq.MT19937(seed), OracleMT(seed)
        # a few calls in a row on one stream, as a decode loop would
        for call in range(3):
            got = kq.speculative_decide_mt(draft, q, p, orders, g)
            want = oracle_decide_mt(draft, q, p, orders, o)
            assert got == want, (trial, call, got, want)
            outcomes.add(got[0] == k)
        assert int(g.u32(1)[0]) == o.next_u32(), f"trial {trial}: streams diverged"
    if k:
        assert outcomes == {True, False}, "every trial took the same branch"


def test_decide_mt_errors_draw_nothing_and_write_nothing():
    lib = kq.load()
    rng = np.random.default_rng(5)
    draft, q, p, orders = random_case(rng, 12, 3)
    dt = np.ascontiguousarray(draft, dtype=np.int32)
    vp = ctypes.c_void_p
    g = kq.MT19937(77)
    acc, nxt = ctypes.c_int32(-5), ctypes.c_int32(-6)

    def call(k=3, tokens=dt, n=12, dr=q, tr=p, od=orders, state=None, a=True, b=True):
        return lib.kq_speculative_decide_mt(
            k, vp(tokens.ctypes.data) if tokens is not None else None, n,
            vp(dr.ctypes.data) if dr is not None else None, vp(tr.ctypes.data) if tr is not None else None,
            vp(od.ctypes.data) if od is not None else None,
            ctypes.byref(g.state) if state is None else state,
            ctypes.byref(acc) if a else None, ctypes.byref(nxt) if b else None)

    bad_tok = dt.copy()
    bad_tok[1] = 12
    assert call(tokens=bad_tok) == TOKEN
    assert call(k=16) == SHAPE
    assert call(k=-1) == SHAPE
    assert call(n=0) == SHAPE
    assert call(tr=None) == NULL
    assert call(od=None) == NULL
    assert call(a=False) == NULL
    assert call(b=False) == NULL
    assert call(state=ctypes.POINTER(kq.MT19937State)()) == NULL
    corrupt = kq.MT19937(77)
    corrupt.state.index = 625
    before = bytes(corrupt.state)
    assert lib.kq_speculative_decide_mt(3, vp(dt.ctypes.data), 12, vp(q.ctypes.data), vp(p.ctypes.data),
                                        vp(orders.ctypes.data), ctypes.byref(corrupt.state),
                                        ctypes.byref(acc), ctypes.byref(nxt)) == SHAPE
    assert bytes(corrupt.state) == before
    # a rejection whose residual and target row hold no positive value to draw
    zero_p = p.copy()
    zero_p[0] = 0.0
    assert call(tr=zero_p) == SHAPE
    assert (acc.value, nxt.value) == (-5, -6)
    assert int(g.u32(1)[0]) == OracleMT(77).next_u32(), "a refused call moved the stream"


def test_generator_argument_errors():
    lib = kq.load()
    st = kq.MT19937State()
    assert lib.kq_mt19937_seed(None, 1) == NULL
    assert lib.kq_mt19937_seed(ctypes.byref(st), 1) == 0
    out = np.zeros(4, dtype=np.uint32)
    assert lib.kq_mt19937_u32(ctypes.byref(st), None, 4) == NULL
    assert lib.kq_mt19937_u32(ctypes.byref(st), None, 0) == 0
    assert lib.kq_mt19937_u32(ctypes.byref(st), ctypes.c_void_p(out.ctypes.data), -1) == SHAPE
    assert lib.kq_mt19937_uniform_f32(None, ctypes.c_void_p(out.ctypes.data), 1) == NULL
    st.index = 700
    assert lib.kq_mt19937_u32(ctypes.byref(st), ctypes.c_void_p(out.ctypes.data), 1) == SHAPE
    assert lib.kq_mt19937_uniform_f32(ctypes.byref(st), ctypes.c_void_p(out.ctypes.data), 1) == SHAPE
    assert st.index == 700 and not out.any()

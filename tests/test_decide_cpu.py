"""The library's host decision of the stochastic verify (kq_speculative_decide)
against the oracle, bit for bit on the same fp32 inputs (no GPU needed), and
its argument checks (all before the first draw)."""
import ctypes

import numpy as np
import pytest

from oracle.stochastic import speculative_decide as oracle_decide
from quant_verify_gemv_amd import lib as kq

NULL, SHAPE, TOKEN = 1, 2, 4


def random_case(rng, n, k, peaked=False):
    z = rng.normal(size=(k + 1, n)) * (4.0 if peaked else 1.0)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    y = rng.normal(size=(k, n)) * (4.0 if peaked else 1.0)
    q = np.exp(y - y.max(axis=1, keepdims=True))
    q = (q / q.sum(axis=1, keepdims=True)).astype(np.float32)
    # proposals drawn from the draft rows, as a draft would
    draft = [int(rng.choice(n, p=q[i] / q[i].sum())) for i in range(k)]
    orders = np.stack([rng.permutation(n) for _ in range(k + 1)]).astype(np.int32)
    u = rng.random(k + 1).astype(np.float32)
    return draft, q, p, orders, u


@pytest.mark.parametrize("n,k", [(5, 3), (64, 7), (1000, 15), (7, 0)])
def test_decide_matches_oracle_bitwise(n, k):
    rng = np.random.default_rng(n * 31 + k)
    seen = set()
    for trial in range(300 if n < 1000 else 40):
        draft, q, p, orders, u = random_case(rng, n, k, peaked=trial % 2 == 1)
        got = kq.speculative_decide(draft, q, p, orders, u)
        want = oracle_decide(draft, q, p, orders, u)
        assert got == want, (trial, got, want)
        seen.add(got[0])
    if k:
        assert len(seen) > 1, "every trial took the same branch"


def test_decide_one_hot_is_greedy():
    n, k = 6, 4
    rng = np.random.default_rng(9)
    for _ in range(200):
        am = rng.integers(0, n, k + 1)
        draft = [int(am[i]) if rng.random() < 0.7 else int(rng.integers(n)) for i in range(k)]
        p = np.eye(n, dtype=np.float32)[am]
        q = np.eye(n, dtype=np.float32)[draft]
        orders = np.tile(np.arange(n, dtype=np.int32), (k + 1, 1))
        acc, nxt = kq.speculative_decide(draft, q, p, orders, rng.random(k + 1).astype(np.float32) * 0.999)
        want = next((i for i in range(k) if draft[i] != am[i]), k)
        assert (acc, nxt) == (want, int(am[want]))


def test_decide_argument_errors():
    lib = kq.load()
    n, k = 4, 2
    p = np.full((k + 1, n), 0.25, np.float32)
    q = np.full((k, n), 0.25, np.float32)
    o = np.tile(np.arange(n, dtype=np.int32), (k + 1, 1))
    u = np.full(k + 1, 0.5, np.float32)
    d = np.array([1, 2], np.int32)
    acc, nxt = ctypes.c_int32(), ctypes.c_int32()
    vp = ctypes.c_void_p

    def call(k=k, d=d, n=n, q=q, p=p, o=o, u=u, a=True):
        return lib.kq_speculative_decide(k, vp(d.ctypes.data) if d is not None else None, n,
                                         vp(q.ctypes.data) if q is not None else None,
                                         vp(p.ctypes.data) if p is not None else None,
                                         vp(o.ctypes.data) if o is not None else None,
                                         vp(u.ctypes.data) if u is not None else None,
                                         ctypes.byref(acc) if a else None, ctypes.byref(nxt))
    assert call() == 0
    assert call(p=None) == NULL and call(o=None) == NULL and call(u=None) == NULL and call(a=False) == NULL
    assert call(d=None) == NULL and call(q=None) == NULL
    assert call(k=-1) == SHAPE and call(k=16) == SHAPE and call(n=0) == SHAPE
    assert call(d=np.array([1, 4], np.int32)) == TOKEN
    bad = o.copy()
    bad[2, 3] = 9  # row k is the one sampled when every proposal is accepted
    acc.value = nxt.value = -7
    assert call(o=bad) == TOKEN and acc.value == -7 and nxt.value == -7  # no output on error
    unread = o.copy()
    unread[0, 1] = 9  # a row that is not sampled is not read
    assert call(o=unread) == 0 and acc.value == k
    # a row to sample without any positive probability
    assert call(k=0, p=np.zeros((1, n), np.float32), o=o[:1], u=u[:1]) == 0  # bonus walks every token
    zero = p.copy()
    zero[0] = 0
    qq = q.copy()
    qq[0] = 0.5
    assert call(p=zero, q=qq, u=np.array([0.9, 0.5, 0.5], np.float32)) == SHAPE


def test_softmax_argument_errors_before_any_hip_call():
    lib = kq.load()
    FAKE = 0x7F0000000000
    assert kq.softmax_workspace_bytes(0, 10) == 0 and kq.softmax_workspace_bytes(16, 0) == 0
    assert kq.softmax_workspace_bytes(16, 131072) >= 16 * 32 * 8
    ws = kq.softmax_workspace_bytes(16, 131072)
    assert lib.kq_softmax_rows(None, 16, 131072, 1.0, 0.0, FAKE, FAKE, ws, None) == NULL
    assert lib.kq_softmax_rows(FAKE, 16, 131072, 0.0, 0.0, FAKE, FAKE, ws, None) == SHAPE
    assert lib.kq_softmax_rows(FAKE, 16, 131072, 1.0, -1.0, FAKE, FAKE, ws, None) == SHAPE
    assert lib.kq_softmax_rows(FAKE, 16, 131072, float("inf"), 0.0, FAKE, FAKE, ws, None) == SHAPE
    assert lib.kq_softmax_rows(FAKE, 0, 131072, 1.0, 0.0, FAKE, FAKE, ws, None) == SHAPE
    assert lib.kq_softmax_rows(FAKE + 2, 16, 131072, 1.0, 0.0, FAKE, FAKE, ws, None) == 3
    assert lib.kq_softmax_rows(FAKE, 16, 131072, 1.0, 0.0, FAKE, FAKE, ws - 1, None) == 5


@pytest.mark.parametrize("n,k", [(5, 3), (64, 7), (1000, 15), (7, 0)])
def test_two_step_decision_matches_oracle(n, k):
    """kq_speculative_first_reject on p_i[d_i], q_i[d_i] alone, then
    kq_speculative_resample on the one row pair (or target row k) it names,
    equals the oracle's decision on the full rows, bit for bit."""
    rng = np.random.default_rng(n * 37 + k)
    for trial in range(200 if n < 1000 else 30):
        draft, q, p, orders, u = random_case(rng, n, k, peaked=trial % 2 == 1)
        p_at = np.array([p[i, d] for i, d in enumerate(draft)], dtype=np.float32)
        q_at = np.array([q[i, d] for i, d in enumerate(draft)], dtype=np.float32)
        j = kq.speculative_first_reject(p_at, q_at, u[:k])
        if j < k:
            tok = kq.speculative_resample(p[j], q[j], orders[j], u[j + 1])
        else:
            tok = kq.speculative_resample(p[k], None, orders[k], u[k])
        assert (j, tok) == oracle_decide(draft, q, p, orders, u), trial


def test_two_step_decision_errors():
    lib = kq.load()
    pos = ctypes.c_int32(-7)
    one = np.ones(4, dtype=np.float32)
    vp = lambda a: ctypes.c_void_p(a.ctypes.data)
    assert lib.kq_speculative_first_reject(2, None, vp(one), vp(one), ctypes.byref(pos)) == NULL
    assert lib.kq_speculative_first_reject(16, vp(one), vp(one), vp(one), ctypes.byref(pos)) == SHAPE
    assert lib.kq_speculative_first_reject(0, None, None, None, ctypes.byref(pos)) == 0 and pos.value == 0
    # a NaN probability rejects; q <= 0 accepts
    nan = np.array([np.nan, 1.0], dtype=np.float32)
    assert kq.speculative_first_reject(nan, np.ones(2, np.float32), np.zeros(2, np.float32)) == 0
    assert kq.speculative_first_reject(np.zeros(2, np.float32), np.zeros(2, np.float32), np.full(2, 0.99, np.float32)) == 2
    tok = ctypes.c_int32(-7)
    p = np.array([0.5, 0.5, 0.0], dtype=np.float32)
    bad = np.array([0, 3, 1], dtype=np.int32)
    assert lib.kq_speculative_resample(3, vp(p), None, vp(bad), ctypes.c_float(0.1), ctypes.byref(tok)) == TOKEN
    assert lib.kq_speculative_resample(0, vp(p), None, vp(bad), ctypes.c_float(0.1), ctypes.byref(tok)) == SHAPE
    zero = np.zeros(3, dtype=np.float32)
    order = np.array([2, 0, 1], dtype=np.int32)
    # residual of p against itself is zero: falls back to p, whose walk skips the zero entry
    assert kq.speculative_resample(p, p, order, 0.75) == 1
    assert lib.kq_speculative_resample(3, vp(zero), vp(zero), vp(order), ctypes.c_float(0.1), ctypes.byref(tok)) == SHAPE
    assert tok.value == -7, "written on an error"
    assert kq.speculative_resample(p, None, order, 0.25) == 0


def test_decide_edge_cases_match_oracle():
    """The library's decision on the boundary cases the oracle's pins fix:
    a draw equal to the acceptance probability accepts; a zero residual
    resamples from the target row; a walk that rounding lets run off the end
    returns the last token that has residual mass, never the rejected one."""
    o4 = np.array([list(range(4))] * 2, dtype=np.int32)
    q = np.array([[0.5, 0.5, 0.0, 0.0]], dtype=np.float32)
    p = np.array([[0.25] * 4, [0.1, 0.2, 0.3, 0.4]], dtype=np.float32)
    half_up = float(np.nextafter(np.float32(0.5), np.float32(1)))
    r = [14.628571510314941, 21.571428298950195, 27.14285659790039]
    p5 = np.array([[r[0], r[1], r[2], 0.0, 1.0], [0.2] * 5], dtype=np.float32)
    q5 = np.array([[0.0, 0.0, 0.0, 0.0, 2.0]], dtype=np.float32)
    o5 = np.array([list(range(5))] * 2, dtype=np.int32)
    top = float(np.float32(1.0) - np.float32(2.0 ** -24))
    p3 = np.array([[0.1, 0.2, 0.3, 0.4]] * 3, dtype=np.float32)
    q_big = np.array([[0.5] * 4, [0.25] * 4], dtype=np.float32)
    o3 = np.array([list(range(4))] * 3, dtype=np.int32)
    cases = [([0], q, p, o4, [0.5, 0.05], (1, 0)), ([0], q, p, o4, [half_up, 0.05], (0, 2)),
             ([4], q5, p5, o5, [0.9, top], (0, 2)), ([3, 0], q_big, p3, o3, [0.9, 0.35, 0.5], (0, 2))]
    for draft, qq, pp, oo, u, want in cases:
        uu = np.array(u, dtype=np.float32)
        assert oracle_decide(draft, qq, pp, oo, uu) == want
        assert kq.speculative_decide(draft, qq, pp, oo, uu) == want

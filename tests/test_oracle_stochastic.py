"""Pins of the stochastic-verify oracle (oracle/stochastic.py) against closed
forms, hand cases, the greedy limit and the exactness theorem of the accept /
residual rule (the emitted token is distributed as the target's row)."""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle.stochastic import sample_ordered, softmax_rows, speculative_decide


# ------------------------------------------------------------------ softmax

def test_softmax_closed_forms():
    assert np.allclose(softmax_rows(np.zeros((2, 8))), 1 / 8, rtol=0, atol=1e-15)
    p = softmax_rows(np.array([[0.0, math.log(2.0)]]))
    assert np.allclose(p, [[1 / 3, 2 / 3]], rtol=0, atol=1e-15)
    # temperature 2 halves the log-odds: [0, ln 4] at T = 2 equals [0, ln 2] at T = 1
    assert np.allclose(softmax_rows(np.array([[0.0, math.log(4.0)]]), temperature=2.0), p, atol=1e-15)
    # soft cap: a huge logit is capped at the cap, so p = e^c / (e^c + 1)
    c = 30.0
    q = softmax_rows(np.array([[1e6, 0.0]]), soft_cap=c)
    assert abs(q[0, 1] - 1.0 / (math.exp(c) + 1.0)) < 1e-25
    # a cap far above every logit changes nothing measurable
    rng = np.random.default_rng(0)
    L = rng.normal(size=(3, 50)) * 5
    assert np.allclose(softmax_rows(L, soft_cap=1e9), softmax_rows(L), rtol=1e-12, atol=0)


def test_softmax_invariants():
    rng = np.random.default_rng(1)
    L = rng.normal(size=(4, 1000)) * 20
    p = softmax_rows(L)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert np.allclose(softmax_rows(L + 123.0), p, rtol=1e-12, atol=0)   # shift invariance
    # ratios are exp of logit differences
    i, j = 3, 7
    assert np.allclose(p[:, i] / p[:, j], np.exp(L[:, i] - L[:, j]), rtol=1e-9)
    # a very low temperature concentrates the row on its argmax
    cold = softmax_rows(L, temperature=1e-4)
    assert np.array_equal(cold.argmax(axis=1), L.argmax(axis=1))
    assert np.all(cold.max(axis=1) > 1 - 1e-12)
    with pytest.raises(ValueError):
        softmax_rows(L, temperature=0.0)


# ----------------------------------------------------------- ordered sampling

def test_sample_ordered_hand_cases():
    prob = np.array([0.25, 0.25, 0.5], dtype=np.float32)
    assert [sample_ordered(prob, [0, 1, 2], u) for u in (0.0, 0.1, 0.25, 0.3, 0.6, 0.999)] == [0, 0, 1, 1, 2, 2]
    # the order decides which token a draw lands on
    assert [sample_ordered(prob, [2, 1, 0], u) for u in (0.1, 0.5, 0.6, 0.8)] == [2, 1, 1, 0]
    # rounding that leaves the draw above the total returns the last token of the order
    assert sample_ordered(np.array([0.3, 0.3], dtype=np.float32), [1, 0], 0.99) == 0


def test_sample_ordered_frequencies_match_probabilities():
    rng = np.random.default_rng(2)
    prob = rng.random(7).astype(np.float32)
    prob = (prob / prob.sum()).astype(np.float32)
    order = list(rng.permutation(7))
    g = 20000
    counts = np.zeros(7)
    for i in range(g):
        counts[sample_ordered(prob, order, (i + 0.5) / g)] += 1
    assert np.allclose(counts / g, prob, atol=2e-4)


# ------------------------------------------------------------------- decide

def one_hot(n, t):
    v = np.zeros(n, np.float32)
    v[t] = 1
    return v


def test_decide_one_hot_rows_reduce_to_the_greedy_rule():
    """Temperature-0 limit: one-hot target rows (the argmax) and one-hot draft
    rows (the proposal). Every draft and argmax vector for N = 4, k = 3, a
    few uniform draws each, against the oracle's greedy accept."""
    n, k = 4, 3
    rng = np.random.default_rng(3)
    orders = np.array([list(range(n))] * (k + 1))
    for draft in itertools.product(range(n), repeat=k):
        for am in itertools.product(range(n), repeat=k + 1):
            q = np.stack([one_hot(n, t) for t in draft])
            p = np.stack([one_hot(n, t) for t in am])
            u = rng.random(k + 1) * 0.999
            assert speculative_decide(draft, q, p, orders, u) == oracle.accept(draft, am)


def test_decide_output_is_distributed_as_the_target():
    """The exactness theorem: with the proposal d drawn from the draft row q0,
    the token emitted at position 0 (d if accepted, else the residual draw)
    is distributed as the target row p0. Integrated over d and over a
    stratified grid of the two draws that decide position 0."""
    rng = np.random.default_rng(4)
    n, k, g = 5, 2, 120
    for trial in range(3):
        p = rng.dirichlet(np.ones(n), size=k + 1).astype(np.float32)
        q = rng.dirichlet(np.ones(n), size=k).astype(np.float32)
        orders = np.array([rng.permutation(n) for _ in range(k + 1)])
        out = np.zeros(n)
        for d0 in range(n):
            draft = [d0, int(rng.integers(n))]
            counts = np.zeros(n)
            for a in range(g):
                for b in range(g):
                    u = [(a + 0.5) / g, (b + 0.5) / g, 0.5]
                    acc, nxt = speculative_decide(draft, q, p, orders, u)
                    counts[d0 if acc >= 1 else nxt] += 1
            out += q[0, d0] * counts / (g * g)
        assert np.allclose(out, p[0], atol=0.02), (trial, out, p[0])


def test_decide_special_cases():
    n = 4
    orders = np.array([list(range(n))] * 3)
    p = np.array([[0.1, 0.2, 0.3, 0.4]] * 3, dtype=np.float32)
    # identical rows: every proposal is accepted (p/q = 1), the bonus comes from row k
    assert speculative_decide([3, 1], p[:2], p, orders, [0.9999, 0.9999, 0.05]) == (2, 0)
    assert speculative_decide([3, 1], p[:2], p, orders, [0.5, 0.5, 0.95]) == (2, 3)
    # a draft probability of zero counts as certain acceptance
    q0 = np.array([[0.5, 0.5, 0.0, 0.0], [0.25] * 4], dtype=np.float32)
    assert speculative_decide([2, 0], q0, p, orders, [0.9999, 0.0, 0.5])[0] >= 1
    # a rejection whose residual sums to zero draws from the target row itself
    q_big = np.array([[0.5, 0.5, 0.5, 0.5], [0.25] * 4], dtype=np.float32)
    acc, nxt = speculative_decide([3, 0], q_big, p, orders, [0.9, 0.05, 0.5])
    assert acc == 0 and nxt == sample_ordered(p[0], list(range(n)), 0.05) == 0
    # ... and at a draw where walking the draft row instead would differ
    # (target cumulative 0.1, 0.3, 0.6: token 2; draft cumulative 0.5: token 0)
    assert speculative_decide([3, 0], q_big, p, orders, [0.9, 0.35, 0.5]) == (0, 2)
    # geometry is checked before any draw
    with pytest.raises(ValueError):
        speculative_decide([1], p[:1], p[:1], orders[:2], [0.5, 0.5])
    with pytest.raises(ValueError):
        speculative_decide([7], p[:1], p[:2], orders[:2], [0.5, 0.5])



def test_decide_accepts_a_draw_equal_to_the_acceptance():
    """The page's rule accepts when the draw is at most the acceptance
    probability: p/q = 0.25/0.5 = 0.5 exactly, and the draw 0.5 accepts
    (the bonus then comes from row 1); a strict comparison would reject and
    resample from the residual (tokens 2 and 3)."""
    orders = np.array([list(range(4))] * 2)
    q = np.array([[0.5, 0.5, 0.0, 0.0]], dtype=np.float32)
    p = np.array([[0.25] * 4, [0.1, 0.2, 0.3, 0.4]], dtype=np.float32)
    assert speculative_decide([0], q, p, orders, [0.5, 0.05]) == (1, 0)
    assert speculative_decide([0], q, p, orders, [np.nextafter(np.float32(0.5), np.float32(1)), 0.05]) == (0, 2)


def test_decide_never_emits_a_token_without_residual_mass():
    """After a rejection the replacement is drawn from the renormalised
    residual max(p - q, 0), so a token whose residual is zero is never
    emitted, even when fp32 rounding leaves the walk's sum below the draw.
    Here the residual is [r0, r1, r2, 0, 0] whose normalised fp32 walk sums
    to exactly 1 - 2^-24, the largest draw, so that draw runs off the end
    and the last token with residual mass (2) is the answer; tokens 3
    (p = 0) and 4 (the rejected proposal, p < q) have none."""
    r = [14.628571510314941, 21.571428298950195, 27.14285659790039]
    p = np.array([[r[0], r[1], r[2], 0.0, 1.0], [0.2] * 5], dtype=np.float32)
    q = np.array([[0.0, 0.0, 0.0, 0.0, 2.0]], dtype=np.float32)
    orders = np.array([list(range(5))] * 2)
    top = float(np.float32(1.0) - np.float32(2.0 ** -24))
    resid = np.maximum(p[0] - q[0], np.float32(0.0)).astype(np.float32)
    total = np.float32(0.0)
    for v in resid:
        total = np.float32(total + v)
    c = np.float32(0.0)
    for v in (resid / total).astype(np.float32):
        c = np.float32(c + v)
    assert c == np.float32(top)  # the walk cannot pass the top draw
    assert speculative_decide([4], q, p, orders, [0.9, top]) == (0, 2)

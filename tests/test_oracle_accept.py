"""Pins for the oracle's greedy accept rule and argmax/flags (CPU only).

The accept/resample rule of muser-book ch. 33 ("Speculation: the local win
and the distributed verdict", section 33.2) is stochastic; the verify step
built here is its temperature-0 limit. Pins: brute force over every draft and
argmax vector for a tiny vocabulary, the stochastic rule re-implemented from
the page's description with one-hot distributions, and the page's own verify
arithmetic in section 33.5 (tests/golden/spec_bar_ch33_s33_5.json).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _longest_prefix(draft, am):
    k = len(draft)
    for length in range(k, -1, -1):  # check every prefix length, longest first
        if all(draft[i] == am[i] for i in range(length)):
            return length, am[length]
    raise AssertionError


def test_accept_brute_force_vocab4_k3():
    V, k = 4, 3
    n = 0
    for draft in itertools.product(range(V), repeat=k):
        for am in itertools.product(range(V), repeat=k + 1):
            assert oracle.accept(draft, am) == _longest_prefix(draft, am)
            n += 1
    assert n == 4 ** 3 * 4 ** 4


def test_accept_k0_returns_first_row():
    assert oracle.accept([], [7]) == (0, 7)


def _stochastic_verify(draft, q_rows, p_rows, u_stream):
    """The page's accept/resample procedure, restated: for each proposed
    token accept with probability min(p/q, 1) (always when q <= 0); at the
    first rejection stop and draw the replacement from the renormalised
    positive part of p - q (p itself if that part is empty); if every
    proposal is accepted draw the extra token from the last target row.
    A draw from a distribution walks it in index order until the running sum
    passes u."""
    def sample(dist, u):
        tot = 0.0
        for t, pr in enumerate(dist):
            if pr <= 0:
                continue
            tot += pr
            if u < tot:
                return t
        return max(t for t, pr in enumerate(dist) if pr > 0)

    for i, tok in enumerate(draft):
        q, p = q_rows[i][tok], p_rows[i][tok]
        a = 1.0 if q <= 0 else min(p / q, 1.0)
        if next(u_stream) <= a:
            continue
        res = [max(pp - qq, 0.0) for pp, qq in zip(p_rows[i], q_rows[i])]
        tot = sum(res)
        res = list(p_rows[i]) if tot <= 0 else [r / tot for r in res]
        return i, sample(res, next(u_stream))
    return len(draft), sample(p_rows[-1], next(u_stream))


def test_one_hot_stochastic_rule_reduces_to_greedy():
    g = np.random.default_rng(21)
    V = 9
    for _ in range(3000):
        k = int(g.integers(0, 8))
        am = [int(v) for v in g.integers(0, V, k + 1)]
        draft = [am[i] if g.random() < 0.7 else int(g.integers(0, V)) for i in range(k)]
        p_rows = [[1.0 if t == am[i] else 0.0 for t in range(V)] for i in range(k + 1)]
        q_rows = [[1.0 if t == draft[i] else 0.0 for t in range(V)] for i in range(k)]
        us = iter(g.uniform(1e-12, 1.0 - 1e-12, size=2 * k + 2))
        assert _stochastic_verify(draft, q_rows, p_rows, us) == oracle.accept(draft, am)


def _expected_emitted_by_enumeration(a, k):
    """E[accepted + 1] with IID per-edge acceptance a, enumerating all 2^k
    match/mismatch patterns through the oracle's accept."""
    am = list(range(k + 1))
    tot = 0.0
    for pattern in itertools.product([True, False], repeat=k):
        draft = [am[i] if ok else am[i] + 1000 for i, ok in enumerate(pattern)]
        acc, nxt = oracle.accept(draft, am)
        assert nxt == am[acc]
        hits = sum(pattern)
        tot += (a ** hits) * ((1 - a) ** (k - hits)) * (acc + 1)
    return tot


def test_page_bar_arithmetic_k15():
    gold = json.load(open(os.path.join(GOLDEN, "spec_bar_ch33_s33_5.json")))
    k = gold["verify_length"]
    cycle = (gold["m16_target_wall_ms"] + gold["draft_ms"] + gold["rtt_ms"]
             + gold["capture_ms"] + gold["sparse_q_ms"]) / 1000.0
    # full acceptance: a verify of k drafts emits k + 1 tokens
    assert _expected_emitted_by_enumeration(1.0, k) == k + 1
    assert (k + 1) / cycle == pytest.approx(gold["full_acceptance_tok_s"], abs=0.01)
    # the per-edge acceptance the page says the 107.9 bar needs
    a = gold["required_acceptance"]
    e = _expected_emitted_by_enumeration(a, k)
    assert e == pytest.approx((1 - a ** (k + 1)) / (1 - a), rel=1e-12)
    assert e / cycle == pytest.approx(gold["bar_tok_s"], abs=0.05)
    cycle95 = cycle + (gold["m16_target_wall_p95_ms"] - gold["m16_target_wall_ms"]) / 1000.0
    a95 = gold["required_acceptance_p95"]
    assert ((1 - a95 ** (k + 1)) / (1 - a95)) / cycle95 == pytest.approx(gold["bar_tok_s"], abs=0.05)
    # 16 x 33,280 fp32 capture rows are the page's capture byte count
    assert 16 * synthetic.FC_IN * 4 == gold["capture_bytes"]


def test_injected_drafts_follow_mismatch_chain():
    # E[accepted] = sum_i prod_{j<=i} (1 - p_j); P(all k accepted) = prod (1 - p_j)
    k, V, trials = 15, 50, 20000
    p = synthetic.mismatch_probs(k)
    surv = np.cumprod(1 - p)
    e_acc, p_all = float(np.sum(surv)), float(surv[-1])
    assert e_acc == pytest.approx(3.51, abs=0.01)
    assert p_all == pytest.approx(0.018, abs=0.002)
    g = np.random.default_rng(5)
    accs = []
    for t in range(trials):
        am = [int(v) for v in g.integers(0, V, k + 1)]
        draft = synthetic.inject_mismatches(am[:k], V, seed=1000 + t)
        for i in range(k):
            assert 0 <= draft[i] < V
        acc, nxt = oracle.accept(draft, am)
        assert nxt == am[acc]
        accs.append(acc)
    accs = np.array(accs)
    se = accs.std() / np.sqrt(trials)
    assert abs(accs.mean() - e_acc) < 4 * se
    assert abs(np.mean(accs == k) - p_all) < 4 * np.sqrt(p_all * (1 - p_all) / trials)


def test_argmax_ties_lowest_index_and_signed_zero():
    L = np.array([[1.0, 3.0, 3.0, 2.0],
                  [-0.0, 0.0, -1.0, -0.0],
                  [0.0, -0.0, -5.0, -1.0]])
    A = np.zeros_like(L)
    am, nc = oracle.argmax_flags(L, A)
    assert list(am) == [1, 0, 0]
    # exact ties are candidates even with zero tolerance
    assert list(nc) == [1, 2, 1]


def test_argmax_flags_and_candidates_hand_cases():
    L = np.array([[10.0, 9.0, 9.9, 0.0, 9.99]])
    A = np.array([[100.0, 100.0, 100.0, 100.0, 100.0]])
    # tol_j = 1e-2 * A_j = 1; gap <= tol_best + tol_j = 2 -> {1, 2, 4}
    am, nc = oracle.argmax_flags(L, A, rel=1e-2)
    assert am[0] == 0 and nc[0] == 3
    assert list(oracle.candidates(L[0], A[0], 0, rel=1e-2)) == [1, 2, 4]
    am, nc = oracle.argmax_flags(L, A, rel=1e-4)
    assert am[0] == 0 and nc[0] == 1  # only 9.99 within 0.02
    assert list(oracle.candidates(L[0], A[0], 0, rel=1e-4)) == [4]


def test_flag_tolerance_is_the_sum_of_both_rows():
    """The flag rule sums both rows' tolerances: j is a candidate iff
    L[i*] - L[j] <= rel (A[i*] + A[j]). With rel = 1e-3 the tolerances are
    0.3, 0.1, 0.01, 1.0, 0.1; the gaps 0.35, 0.305 and 1.2 fit only the sum
    (each is above either row's tolerance alone), the gap 0.5 fits neither."""
    L = np.array([[5.0, 4.65, 4.695, 3.8, 4.5]])
    A = np.array([[300.0, 100.0, 10.0, 1000.0, 100.0]])
    am, nc = oracle.argmax_flags(L, A, rel=1e-3)
    assert am[0] == 0 and nc[0] == 3
    assert list(oracle.candidates(L[0], A[0], 0, rel=1e-3)) == [1, 2, 3]


def test_argmax_through_gemv_duplicated_rows():
    n, k = 32, 512
    w = synthetic.q4k_matrix(n, k, seed=30)
    x = synthetic.activations(4, k, seed=31)
    L, A = oracle.gemv_rows(w, k, x)
    am, _ = oracle.argmax_flags(L, A)
    for m in range(4):
        b = int(am[m])
        for dup in (0, n - 1):
            if dup == b:
                continue
            w2 = w.copy()
            w2[dup] = w[b]  # duplicated weight rows give bit-identical logits
            L2, A2 = oracle.gemv_rows(w2, k, x[m:m + 1])
            assert L2[0, dup] == L2[0, b]
            am2, nc2 = oracle.argmax_flags(L2, A2)
            assert am2[0] == min(dup, b)  # the lowest index of the tie wins
            assert max(dup, b) in oracle.candidates(L2[0], A2[0], int(am2[0]))

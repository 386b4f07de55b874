"""Parity checks of the HIP path against the oracle.

Criteria (the tolerance the logits are held to is 1e-4 * sum_k |w_k x_k|,
fp32 accumulation; argmax and accepted length are compared exactly except
where the oracle's top-2 gap is within the two elements' tolerances):

* logits: |G - L| <= REL * A for every element (L, A from the oracle, fp64);
* argmax: unflagged rows must equal the oracle's index; flagged rows must
  pick the oracle's index or one of its candidates;
* accept: the GPU's (accepted, next) must equal the rule applied to the GPU's
  own argmaxes, and equal the oracle's when no row up to the oracle's
  accepted position is flagged.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

REL = oracle.REL_TOL


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_logits(G: np.ndarray, L: np.ndarray, A: np.ndarray, rel: float = REL, what: str = ""):
    G = np.asarray(G, dtype=np.float64)
    assert G.shape == L.shape, (G.shape, L.shape)
    assert np.all(np.isfinite(G)), f"{what}: non-finite GPU logits"
    err = np.abs(G - L)
    tol = rel * A
    bad = err > tol
    ratio = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} logits outside tolerance; first {tuple(i)}: "
                             f"gpu {G[tuple(i)]!r} oracle {L[tuple(i)]!r} tol {tol[tuple(i)]!r}")
    return ratio


def check_argmax(g_am, L, A, rel: float = REL, what: str = ""):
    o_am, o_nc = oracle.argmax_flags(L, A, rel)
    g_am = np.asarray(g_am)
    flagged = []
    for m in range(L.shape[0]):
        if o_nc[m] == 0:
            assert int(g_am[m]) == int(o_am[m]), f"{what}: row {m} argmax {g_am[m]} != oracle {o_am[m]}"
        else:
            cands = set(int(c) for c in oracle.candidates(L[m], A[m], int(o_am[m]), rel)) | {int(o_am[m])}
            assert int(g_am[m]) in cands, f"{what}: row {m} argmax {g_am[m]} not in candidate set"
            flagged.append(m)
    return o_am, o_nc, flagged


def check_accept(g_acc, g_next, draft, g_am, o_am, o_nc, what: str = ""):
    acc_g, nxt_g = oracle.accept(draft, [int(v) for v in g_am])
    assert (int(g_acc), int(g_next)) == (acc_g, nxt_g), f"{what}: accept not consistent with GPU argmax"
    acc_o, nxt_o = oracle.accept(draft, [int(v) for v in o_am])
    if not np.any(o_nc[:acc_o + 1] > 0):
        assert (int(g_acc), int(g_next)) == (acc_o, nxt_o), \
            f"{what}: accept ({g_acc},{g_next}) != oracle ({acc_o},{nxt_o})"
    return acc_o, nxt_o

"""Oracle for the stochastic verify (temperature > 0): target probability rows
and the accept / residual-resample decision.

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: only tests/, the smoke
check and the bench's CPU-baseline leg use it. Plain numpy and Python loops,
no code shared with the library.

Passages followed (muser-book chapter 33, "Speculation: the local win and the
distributed verdict", section 33.2, and chapter 32, "Precision across the
handoff", section 32.6):

* The target judges every proposed token against its full probability row
  for that position. The draft token at position i is accepted with
  probability min(p/q, 1), p and q being the target's and the draft's
  probabilities of that token; a draft probability of zero or less counts as
  certain acceptance. One uniform draw per attempted position, in order.
* On the first rejection the replacement is drawn from the residual
  max(p - q, 0), renormalised by its sum; when that sum is not positive the
  target row itself is used. Tokens whose residual is zero are skipped, and
  the draw walks the row in a given token order so that the cumulative sum
  is the same on every run.
* When every proposal is accepted the bonus token is drawn from the last
  row (position k).
* Probabilities are 32-bit floats and the decision is taken in 32-bit
  arithmetic (the sums sequential, in the order written).

Readings where the pages leave a step open (each stated again in the
design notes):

* Uniform draws: u[i] is the draw of the attempt at position i; the draw
  that samples the replacement after a rejection at position i is u[i + 1],
  and the bonus after k acceptances uses u[k] (k + 1 draws cover every
  path). speculative_decide takes them as inputs; speculative_decide_mt
  takes them one at a time from an MT19937 stream (oracle.mt19937, whose
  float conversion is a reading of its own), which is the same rule.
* Sampling walks the order accumulating c = c + p[t] in fp32 and returns the
  first token with u < c; if rounding leaves u >= c after the last token,
  the last token of the order is returned.
* Target rows: p = softmax(z), z = l / T, optionally soft-capped first,
  l -> cap * tanh(l / cap) (cap = 0: no cap). Computed in fp64 here.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

F32 = np.float32


def softmax_rows(logits: np.ndarray, temperature: float = 1.0, soft_cap: float = 0.0) -> np.ndarray:
    """Target probability rows [M, N] (fp64) from logits [M, N]."""
    if not temperature > 0:
        raise ValueError("temperature must be > 0")
    z = np.asarray(logits, dtype=np.float64)
    if soft_cap > 0:
        z = soft_cap * np.tanh(z / soft_cap)
    z = z / temperature
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def _f32_sum(values: np.ndarray) -> np.float32:
    """Sequential fp32 sum, first element first."""
    acc = F32(0.0)
    for v in np.asarray(values, dtype=F32):
        acc = F32(acc + v)
    return acc


def sample_ordered(prob: np.ndarray, order: Sequence[int], u: float) -> int:
    """Walk `order`, accumulating prob[t] in fp32; the first token with
    u < cumulative sum, else the last token of the order."""
    if len(order) == 0:
        raise ValueError("empty order")
    prob = np.asarray(prob, dtype=F32)
    u = F32(u)
    c = F32(0.0)
    for t in order:
        c = F32(c + prob[int(t)])
        if u < c:
            return int(t)
    return int(order[-1])


def speculative_decide(draft: Sequence[int], q_rows: np.ndarray, p_rows: np.ndarray,
                       orders: np.ndarray, uniforms: Sequence[float]) -> Tuple[int, int]:
    """(accepted, next_token) for k = len(draft) proposals.

    q_rows [k, N] and p_rows [k + 1, N] are fp32 probability rows (draft and
    target), orders [k + 1, N] token orders per target row, uniforms k + 1
    draws in [0, 1)."""
    if len(uniforms) != len(draft) + 1:
        raise ValueError("geometry: need k draft rows, k + 1 target rows, orders and uniforms")
    draws = iter(uniforms)
    return _decide(draft, q_rows, p_rows, orders, lambda: F32(next(draws)))


def speculative_decide_mt(draft: Sequence[int], q_rows: np.ndarray, p_rows: np.ndarray,
                          orders: np.ndarray, rng) -> Tuple[int, int]:
    """The same decision taking its draws from a generator (an
    oracle.mt19937.MT19937) in the pages' order, one per attempted proposal
    and one for the token drawn where the decision stops: rng advances by
    accepted + 2 draws after a rejection, by k + 1 when all k are accepted,
    and by none when the geometry is refused."""
    return _decide(draft, q_rows, p_rows, orders, rng.uniform_f32)


def _decide(draft, q_rows, p_rows, orders, draw) -> Tuple[int, int]:
    k = len(draft)
    q_rows = np.asarray(q_rows, dtype=F32)
    p_rows = np.asarray(p_rows, dtype=F32)
    if q_rows.shape[0] != k or p_rows.shape[0] != k + 1 or len(orders) != k + 1:
        raise ValueError("geometry: need k draft rows, k + 1 target rows, orders and uniforms")
    n = p_rows.shape[1]
    if q_rows.shape[1] != n:
        raise ValueError("draft and target rows differ in width")
    for tok in draft:
        if not 0 <= int(tok) < n:
            raise ValueError(f"draft token {int(tok)} outside [0, {n})")
    for i, tok in enumerate(draft):
        tok = int(tok)
        q = q_rows[i, tok]
        p = p_rows[i, tok]
        acceptance = F32(1.0) if q <= 0 else min(F32(p / q), F32(1.0))
        if draw() <= acceptance:
            continue
        residual = np.maximum(p_rows[i] - q_rows[i], F32(0.0)).astype(F32)
        total = _f32_sum(residual)
        if total <= 0:
            residual = p_rows[i].copy()
        else:
            residual = (residual / total).astype(F32)
        order = [int(t) for t in orders[i] if residual[int(t)] > 0]
        return i, sample_ordered(residual, order, draw())
    return k, sample_ordered(p_rows[k], list(orders[k]), draw())

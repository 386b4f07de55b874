"""Pins for the oracle's MT19937 stream and the decision that consumes it
(CPU only).

* The generator: the value the C++ standard fixes for std::mt19937 (the
  10,000th output after default seeding 5489 is 4,123,659,995), and numpy's
  own MT19937 with the reference-code seeding (legacy seeding) word for word
  over several state regenerations, for several seeds.
* The float conversion (a reading): closed forms at the ends and at a few
  exact points.
* The decision with a generator: identical to the decision with explicit
  draws u[i] = the i-th draw of a fresh generator with the same seed, and
  the generator advanced by exactly the draws the pages' order consumes
  (accepted + 2 after a rejection, k + 1 after k acceptances, none when the
  geometry is refused).
"""
import numpy as np
import pytest

from oracle import stochastic
from oracle.mt19937 import MT19937, to_uniform_f32


def test_tenthousandth_output_of_default_seed():
    g = MT19937()
    for _ in range(9999):
        g.next_u32()
    assert g.next_u32() == 4123659995


@pytest.mark.parametrize("seed", [0, 1, 5489, 2 ** 31 + 12345, 2 ** 32 - 1])
def test_matches_numpy_reference_seeding(seed):
    bg = np.random.MT19937()
    bg._legacy_seeding(seed)
    want = bg.random_raw(624 * 3 + 17)
    g = MT19937(seed)
    got = np.array([g.next_u32() for _ in range(len(want))], dtype=np.uint64)
    assert np.array_equal(got, want)


def test_float_conversion_closed_forms():
    assert to_uniform_f32(0) == 0.0
    assert to_uniform_f32(255) == 0.0
    assert to_uniform_f32(256) == np.float32(2.0 ** -24)
    assert to_uniform_f32(0x80000000) == np.float32(0.5)
    assert to_uniform_f32(0xFFFFFFFF) == np.float32(1.0 - 2.0 ** -24)
    assert to_uniform_f32(0xFFFFFFFF) < 1.0
    g = MT19937(7)
    for _ in range(2000):
        u = g.uniform_f32()
        assert u.dtype == np.float32 and 0.0 <= u < 1.0


def _rows(rng, k, n):
    q = rng.dirichlet(np.full(n, 0.3), size=k).astype(np.float32)
    p = rng.dirichlet(np.full(n, 0.3), size=k + 1).astype(np.float32)
    orders = np.stack([rng.permutation(n) for _ in range(k + 1)]).astype(np.int32)
    return q, p, orders


def test_generator_decision_equals_explicit_draws_and_advances_exactly():
    rng = np.random.default_rng(44)
    seen = set()
    for trial in range(300):
        k = int(rng.integers(0, 8))
        n = int(rng.integers(2, 40))
        q, p, orders = _rows(rng, k, n)
        draft = [int(v) for v in rng.integers(0, n, k)]
        seed = int(rng.integers(0, 2 ** 32))
        fresh = MT19937(seed)
        draws = [fresh.uniform_f32() for _ in range(k + 1)]
        g = MT19937(seed)
        acc, tok = stochastic.speculative_decide_mt(draft, q, p, orders, g)
        assert (acc, tok) == stochastic.speculative_decide(draft, q, p, orders, draws)
        used = acc + 2 if acc < k else k + 1
        ref = MT19937(seed)
        for _ in range(used):
            ref.next_u32()
        assert g.next_u32() == ref.next_u32(), f"trial {trial}: generator not advanced by {used} draws"
        seen.add(acc == k)
    assert seen == {True, False}


def test_refused_geometry_consumes_no_draw():
    q, p, orders = _rows(np.random.default_rng(3), 2, 10)
    g = MT19937(99)
    with pytest.raises(ValueError):
        stochastic.speculative_decide_mt([1, 10], q, p, orders, g)  # token outside [0, n)
    with pytest.raises(ValueError):
        stochastic.speculative_decide_mt([1], q, p, orders, g)  # k rows mismatch
    assert g.next_u32() == MT19937(99).next_u32()

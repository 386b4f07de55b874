"""The library's size queries against the shape rule kq.h states, on seeded
random shapes drawn around every limit: k a positive multiple of 256 up to
2^28; 1 <= n < 2^31; 1 <= m <= 64; the weight matrix (rows rounded up to
16) and the staged activations each below 4 GiB; staged blocks of 16,960
bytes per 16-row slice (ceil(m/16) slices: 1 to 4); tiled copies
of ceil(n/16) * (k/256) * 16 * block bytes; launch units of one row group by
one 256-column block. CPU only: the queries make no device call."""
import numpy as np
import pytest

import quant_verify_gemv_amd as kq

STAGE = 16960
LIMIT = 1 << 32
BLOCK = {"q4k": 144, "q5k": 176, "q6k": 210}


def slices(m):
    return -(-m // 16)


def k_ok(k):
    return k > 0 and k % 256 == 0 and k <= 1 << 28


def staged_rule(k, m):
    if not (k_ok(k) and 1 <= m <= 64):
        return 0
    b = (k // 256) * slices(m) * STAGE
    return b if b < LIMIT else 0


def shape_rule(n, k, fmt="q4k"):
    return (1 <= n < 1 << 31 and k_ok(k) and -(-n // 16) * 16 * (k // 256) * BLOCK[fmt] < LIMIT
            and (k // 256) * STAGE < LIMIT)


def draw(rng):
    """One (n, k, m), each from a mixture of ordinary values and values at
    or next to a limit."""
    kb_choice = int(rng.integers(6))
    if kb_choice == 0:
        k = 256 * int(rng.integers(1, 200))
    elif kb_choice == 1:
        k = 256 * (LIMIT // STAGE) + 256 * int(rng.integers(-2, 3))      # staged limit
    elif kb_choice == 2:
        k = (1 << 28) + 256 * int(rng.integers(-2, 3))                   # largest k
    elif kb_choice == 3:
        k = int(rng.integers(-300, 3000))                                # any integer
    elif kb_choice == 4:
        k = 256 * int(np.exp(rng.uniform(0, np.log(1 << 20))))
    else:
        k = 256 * int(rng.integers(1, 4))
    kb = max(1, k // 256)
    n_choice = int(rng.integers(5))
    if n_choice == 0:
        n = int(rng.integers(-2, 400))
    elif n_choice == 1:
        n = int(np.exp(rng.uniform(0, np.log(float(1 << 31)))))
    elif n_choice == 2:
        n = (1 << 31) + int(rng.integers(-3, 3))                         # largest n
    else:
        fmt = ("q4k", "q5k", "q6k")[n_choice % 3]
        n = 16 * (LIMIT // (16 * kb * BLOCK[fmt])) + int(rng.integers(-20, 21))  # weight limit
    m = int(rng.integers(-1, 70))
    return n, k, m


@pytest.mark.parametrize("seed", range(4))
def test_size_queries_follow_the_stated_rule(seed):
    rng = np.random.default_rng(90_000 + seed)
    checked = valid = 0
    for _ in range(1500):
        n, k, m = draw(rng)
        what = f"n={n} k={k} m={m}"
        ok = shape_rule(n, k)
        assert kq.staged_bytes(k, m) == staged_rule(k, m), what
        assert (kq.workspace_bytes(n, k, m) > 0) == (ok and staged_rule(k, m) > 0), what
        assert (kq.scratch_bytes(n, k) > 0) == ok, what
        for fmt, bb in BLOCK.items():
            want = -(-n // 16) * (k // 256) * 16 * bb if shape_rule(n, k, fmt) else 0
            assert kq.tiled_bytes(n, k, fmt) == want, f"{what} {fmt}"
        if ok:
            waves, tpw, wgs, units = kq.launch_geometry(n, k)
            assert (waves, tpw) in ((8, 1), (12, 1), (8, 2)), what
            assert units == -(-n // (16 * waves * tpw)) * (k // 256), what
            assert wgs == min(units, 256), what
            valid += 1
        else:
            with pytest.raises(kq.KQError):
                kq.launch_geometry(n, k)
        checked += 1
    assert valid > 200 and checked - valid > 200  # both sides of the rule were drawn

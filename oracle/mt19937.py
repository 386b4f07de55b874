"""MT19937 draw stream of the stochastic verify (oracle side).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: only tests/, the smoke
check and the bench's CPU-baseline leg use it. Plain Python integers, no
code shared with the library.

Passages followed: muser-book chapter 33, "Speculation: the local win and
the distributed verdict", section 33.2 (every acceptance coin flip and every
resample draw comes from a pinned MT19937 stream, one uniform per attempted
proposal, consumed in order), and chapter 8, "The DFlash draft", section 8.6,
guarantee 1 (the stream reimplements the generator bit for bit, kept apart
from any generic random source).

The generator is the published one (Matsumoto and Nishimura, "Mersenne
Twister: a 623-dimensionally equidistributed uniform pseudo-random number
generator", ACM TOMACS 8(1), 1998), with the initialisation of its 2002
reference code (the one C++'s std::mt19937 and numpy's legacy seeding
use): a 624-word state, the recurrence x[k+624] = x[k+397] xor
((upper bit of x[k] | lower 31 bits of x[k+1]) A), then tempering.

Reading where the pages are silent: the conversion of a 32-bit output to
a float draw. Here u = (w >> 8) * 2^-24 in fp32: the top 24 bits as a
multiple of 2^-24, exact in fp32, so every draw lies in [0, 1 - 2^-24].
"""
from __future__ import annotations

import numpy as np

N = 624
M = 397
MATRIX_A = 0x9908B0DF
UPPER = 0x80000000
LOWER = 0x7FFFFFFF
MASK32 = 0xFFFFFFFF


class MT19937:
    """State: 624 words and the index of the next word to temper (624: the
    block is spent and is regenerated before the next output)."""

    def __init__(self, seed: int = 5489):
        self.seed(seed)

    def seed(self, seed: int) -> None:
        """x[0] = seed, x[i] = 1812433253 (x[i-1] xor (x[i-1] >> 30)) + i
        modulo 2^32."""
        mt = [int(seed) & MASK32]
        for i in range(1, N):
            prev = mt[-1]
            mt.append((1812433253 * (prev ^ (prev >> 30)) + i) & MASK32)
        self.mt = mt
        self.index = N

    def _regenerate(self) -> None:
        mt = self.mt
        for k in range(N):
            y = (mt[k] & UPPER) | (mt[(k + 1) % N] & LOWER)
            v = mt[(k + M) % N] ^ (y >> 1)
            if y & 1:
                v ^= MATRIX_A
            mt[k] = v
        self.index = 0

    def next_u32(self) -> int:
        if self.index >= N:
            self._regenerate()
        y = self.mt[self.index]
        self.index += 1
        y ^= y >> 11
        y ^= (y << 7) & 0x9D2C5680
        y ^= (y << 15) & 0xEFC60000
        y ^= y >> 18
        return y & MASK32

    def uniform_f32(self) -> np.float32:
        return to_uniform_f32(self.next_u32())


def to_uniform_f32(word: int) -> np.float32:
    """The float draw of one 32-bit output: (word >> 8) * 2^-24."""
    return np.float32((int(word) >> 8) * 2.0 ** -24)

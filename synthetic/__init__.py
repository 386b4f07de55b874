"""Seeded synthetic inputs for the Q4_K batched-verify path.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests. It holds no arithmetic of the method itself: it only draws random
bytes and random floats and writes them where the Q4_K super-block format
puts them (two little-endian fp16 words, then 140 free bytes).

Super-block format (256 weights, 144 bytes): bytes 0-1 ``d`` (fp16), bytes
2-3 ``dmin`` (fp16), bytes 4-15 the twelve bytes that carry eight 6-bit scales
and eight 6-bit mins, bytes 16-143 the 128 bytes of 4-bit quants. The pages
name the format only (muser-book ch. 8, section 8.2, "It is kquant"); the
layout is the llama.cpp GGUF one. Because every bit of bytes 4..143 belongs
to exactly one field, uniformly random bytes there give independent uniform
6-bit scales/mins and uniform 4-bit quants.

Workloads follow the shapes the pages give for the target and its DFlash
draft: hidden width 6,656 and the fc projection 33,280 -> 6,656 (muser-book
ch. 8, section 8.2), 16-row verify blocks (ch. 8, section 8.2, block size 16),
a 52-layer target (ch. 33, section 33.1). Vocabulary 131,072 and FFN width
17,920 are the workload's own choices, not from the pages.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Sequence, Tuple

import numpy as np

QK = 256            # weights per super-block
BLOCK_BYTES = 144   # bytes per super-block
HIDDEN = 6656
FFN = 17920
VOCAB = 131072
FC_IN = 5 * HIDDEN  # 33,280: five concatenated target hidden vectors
LAYERS = 52

# Per-position probability that the draft's token differs from the target's
# argmax. One minus the acceptance chain 0.831, 0.786, 0.771, 0.758 reported
# for an MTP depth sweep ("The squeeze", sanctum.run 2026-08-17 post), then
# held flat at the last value because that chain barely decays.
MISMATCH_CHAIN = (0.169, 0.214, 0.229, 0.242)


def _seq(seed: int, stream: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([int(seed), int(stream)])


def q4k_bytes_per_row(k: int) -> int:
    if k % QK:
        raise ValueError(f"K={k} is not a multiple of {QK}")
    return (k // QK) * BLOCK_BYTES


_SM_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_SM_M1 = np.uint64(0xBF58476D1CE4E5B9)
_SM_M2 = np.uint64(0x94D049BB133111EB)
_THREADS = min(8, os.cpu_count() or 1)


def _key(seed: int, stream: int) -> np.uint64:
    return np.uint64(_seq(seed, stream).generate_state(1, np.uint64)[0])


def _splitmix64_fill(out: np.ndarray, start: int, key: np.uint64) -> None:
    """out[i] = SplitMix64 output number start+i+1 of the stream keyed by
    `key` (Steele, Lea & Flood 2014: add the golden-ratio increment, then the
    two xor-shift-multiply mixing rounds)."""
    z = np.arange(start, start + out.shape[0], dtype=np.uint64)
    z += np.uint64(1)
    z *= _SM_GAMMA
    z += key
    z ^= z >> np.uint64(30)
    z *= _SM_M1
    z ^= z >> np.uint64(27)
    z *= _SM_M2
    z ^= z >> np.uint64(31)
    out[:] = z


def random_u64(count: int, seed: int, stream: int) -> np.ndarray:
    """`count` uniformly distributed 64-bit words, deterministic in (seed,
    stream), generated in parallel chunks."""
    key = _key(seed, stream)
    out = np.empty(count, dtype=np.uint64)
    chunk = 1 << 20
    starts = range(0, count, chunk)
    if count <= chunk or _THREADS == 1:
        for s0 in starts:
            _splitmix64_fill(out[s0:s0 + chunk], s0, key)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(lambda s0: _splitmix64_fill(out[s0:s0 + chunk], s0, key), starts))
    return out


def q4k_matrix(n: int, k: int, seed: int, d_range=(0.001, 0.05)) -> np.ndarray:
    """Random Q4_K matrix of N rows x K weights as uint8 [N, K/256*144].

    Bytes 4..143 of every block are uniform random bytes; d and dmin are
    drawn ~U(d_range) in float64 (53-bit uniforms) and rounded to fp16
    (numpy's conversion rounds to nearest even).
    """
    if k % QK:
        raise ValueError(f"K={k} is not a multiple of {QK}")
    nb = n * (k // QK)
    blocks = random_u64(nb * (BLOCK_BYTES // 8), seed, 0).view(np.uint8).reshape(nb, BLOCK_BYTES)
    lo, hi = d_range
    step = 1 << 22
    for b0 in range(0, nb, step):
        b1 = min(nb, b0 + step)
        u = random_u64(2 * (b1 - b0), seed * 1000003 + b0 // step, 1)
        uf = (u >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        dd = (lo + (hi - lo) * uf).astype(np.float16)
        blocks[b0:b1, 0:4] = dd.view(np.uint8).reshape(b1 - b0, 4)
    return blocks.reshape(n, (k // QK) * BLOCK_BYTES)


def q4k_matrix_centred(n: int, k: int, seed: int, d_range=(0.001, 0.05), centre: float = 7.5) -> np.ndarray:
    """Random Q4_K matrix whose weights are centred on zero, as a quantizer
    fitting real weights makes them: every sub-block's min equals its scale
    (m_j = sc_j) and dmin = centre * d (rounded to fp16), so w = d sc_j q -
    dmin m_j is about d sc_j (q - centre), q uniform in [0, 15].

    Built from q4k_matrix's bytes by copying fields where the format keeps
    them: scale/min bytes 0-3 (six low bits: sc_0..3, two top bits: the top
    of sc_4..7) go to bytes 4-7 (m_0..3 and the top of m_4..7), and the low
    nibble of bytes 8-11 (low bits of sc_4..7) to their high nibble (low bits
    of m_4..7)."""
    w = q4k_matrix(n, k, seed, d_range).reshape(-1, BLOCK_BYTES).copy()
    s = w[:, 4:16]
    s[:, 4:8] = s[:, 0:4]
    lo = s[:, 8:12] & np.uint8(0x0F)
    s[:, 8:12] = lo | (lo << np.uint8(4))
    d = w[:, 0:2].copy().view(np.float16).astype(np.float64)
    w[:, 2:4] = (d * centre).astype(np.float16).view(np.uint8)
    return w.reshape(n, (k // QK) * BLOCK_BYTES)


Q5K_BLOCK_BYTES = 176
Q6K_BLOCK_BYTES = 210


def _random_blocks(n: int, k: int, seed: int, block_bytes: int, d_offsets, d_range, stream: int) -> np.ndarray:
    """N x K/256 random blocks of `block_bytes` bytes whose fp16 fields at
    byte offsets `d_offsets` are ~U(d_range) (53-bit uniforms, rounded to
    fp16 to nearest even); every other byte uniform random."""
    if k % QK:
        raise ValueError(f"K={k} is not a multiple of {QK}")
    nb = n * (k // QK)
    words = (nb * block_bytes + 7) // 8
    blocks = random_u64(words, seed, stream).view(np.uint8)[:nb * block_bytes].reshape(nb, block_bytes).copy()
    lo, hi = d_range
    nd = len(d_offsets)
    step = 1 << 22
    for b0 in range(0, nb, step):
        b1 = min(nb, b0 + step)
        u = random_u64(nd * (b1 - b0), seed * 1000003 + b0 // step, stream + 1)
        uf = (u >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        dd = (lo + (hi - lo) * uf).astype(np.float16).view(np.uint8).reshape(b1 - b0, nd, 2)
        for j, off in enumerate(d_offsets):
            blocks[b0:b1, off:off + 2] = dd[:, j, :]
    return blocks.reshape(n, (k // QK) * block_bytes)


def q5k_matrix(n: int, k: int, seed: int, d_range=(0.001, 0.05)) -> np.ndarray:
    """Random Q5_K matrix uint8 [N, K/256*176]: d and dmin (bytes 0..3)
    ~U(d_range) rounded to fp16; scales, fifth bits and nibbles uniform."""
    return _random_blocks(n, k, seed, Q5K_BLOCK_BYTES, (0, 2), d_range, 10)


def q6k_matrix(n: int, k: int, seed: int, d_range=(0.0002, 0.01)) -> np.ndarray:
    """Random Q6_K matrix uint8 [N, K/256*210]: d (bytes 208..209)
    ~U(d_range) rounded to fp16; nibbles, high parts and the signed 8-bit
    scales uniform (a smaller default d keeps |w| = d |sc (q - 32)| <=
    4,096 d in the range of the other formats)."""
    return _random_blocks(n, k, seed, Q6K_BLOCK_BYTES, (208,), d_range, 12)


def kquant_matrix(fmt: str, n: int, k: int, seed: int) -> np.ndarray:
    """Random matrix of format "q4k", "q5k" or "q6k"."""
    return {"q4k": q4k_matrix, "q5k": q5k_matrix, "q6k": q6k_matrix}[fmt](n, k, seed)


def activations(m: int, k: int, seed: int) -> np.ndarray:
    """fp32 activation rows [M, K] ~ N(0, 1)."""
    g = np.random.Generator(np.random.PCG64(_seq(seed, 2)))
    return g.standard_normal((m, k), dtype=np.float32)


def fc_activations(m: int, seed: int, width: int = HIDDEN, parts: int = 5) -> np.ndarray:
    """DFlash fc input rows [M, parts*width]: each row concatenates `parts`
    independent N(0,1) vectors, each scaled to unit RMS (computed in float64,
    then rounded to fp32; no epsilon, no gain)."""
    g = np.random.Generator(np.random.PCG64(_seq(seed, 3)))
    v = g.standard_normal((m, parts, width))
    rms = np.sqrt(np.mean(v * v, axis=2, keepdims=True))
    return (v / rms).astype(np.float32).reshape(m, parts * width)


def mismatch_probs(k: int) -> np.ndarray:
    p = np.empty(k)
    for i in range(k):
        p[i] = MISMATCH_CHAIN[min(i, len(MISMATCH_CHAIN) - 1)]
    return p


def inject_mismatches(target_tokens: Sequence[int], n_vocab: int, seed: int,
                      probs: Sequence[float] | None = None) -> np.ndarray:
    """Draft tokens: a copy of `target_tokens` where position i is replaced,
    with probability probs[i], by a token drawn uniformly from the other
    n_vocab - 1 tokens."""
    t = np.asarray(target_tokens, dtype=np.int64)
    k = t.shape[0]
    p = mismatch_probs(k) if probs is None else np.asarray(probs, dtype=np.float64)
    g = np.random.Generator(np.random.PCG64(_seq(seed, 4)))
    u = g.random(k)
    other = g.integers(0, max(1, n_vocab - 1), size=k)
    out = t.copy()
    if n_vocab < 2:  # no other token exists
        return out.astype(np.int32)
    for i in range(k):
        if u[i] < p[i]:
            out[i] = other[i] + (1 if other[i] >= t[i] else 0)
    return out.astype(np.int32)


def forced_draft(target_tokens: Sequence[int], accepted: int, n_vocab: int) -> np.ndarray:
    """Draft that matches the target on positions < accepted and differs at
    position `accepted` (if accepted < k); later positions are copied."""
    t = np.asarray(target_tokens, dtype=np.int64).copy()
    if accepted < t.shape[0]:
        t[accepted] = (t[accepted] + 1) % n_vocab
    return t.astype(np.int32)


# ---------------------------------------------------------------------------
# Named workloads.

@dataclasses.dataclass(frozen=True)
class Gemv:
    n: int
    k: int
    seed: int

    @property
    def weight_bytes(self) -> int:
        return self.n * q4k_bytes_per_row(self.k)


TINY = dict(n=512, k=1024, m=4, k_draft=3, seed=0)
SQUARE = dict(n=HIDDEN, k=HIDDEN, ms=(1, 2, 4, 8, 16), seed=1)
FC = dict(n=HIDDEN, k=FC_IN, m=16, seed=2)
LM_HEAD = dict(n=VOCAB, k=HIDDEN, m=16, k_draft=15, seed=3)


def stack_matrices(layers: int = LAYERS) -> List[Gemv]:
    """The synthetic target stack: per layer four HIDDEN x HIDDEN matrices,
    two HIDDEN -> FFN and one FFN -> HIDDEN; matrix i of layer l uses seed
    10000 + 8 l + i. (The LM head is the LM_HEAD workload.)"""
    out = []
    for layer in range(layers):
        shapes = [(HIDDEN, HIDDEN)] * 4 + [(FFN, HIDDEN)] * 2 + [(HIDDEN, FFN)]
        for i, (n, k) in enumerate(shapes):
            out.append(Gemv(n=n, k=k, seed=10000 + 8 * layer + i))
    return out


def stack_activation_seed(k: int) -> int:
    """One activation block per distinct K, reused by every stack matrix with
    that K (the stack matrices are independent products, not a chained model)."""
    return 20000 + k


def stack_weight_bytes(layers: int = LAYERS, with_head: bool = True) -> int:
    tot = sum(g.weight_bytes for g in stack_matrices(layers))
    if with_head:
        tot += LM_HEAD["n"] * q4k_bytes_per_row(LM_HEAD["k"])
    return tot

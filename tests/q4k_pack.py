"""Test-side Q4_K packer: builds super-blocks from chosen field values.

Written from the GGUF Q4_K layout independently of the oracle's decoder, so
that a round trip through both catches a mistake in either. 144 bytes per
block: d (fp16), dmin (fp16), 12 bytes of 6-bit scales/mins, 128 bytes of
4-bit quants.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def pack_scales_mins(sc: Sequence[int], mn: Sequence[int]) -> bytes:
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    assert len(sc) == 8 and len(mn) == 8
    assert all(0 <= v < 64 for v in sc + mn)
    s = [0] * 12
    for j in range(4):
        # low six bits: scale j / min j; top two bits: top bits of entry j+4
        s[j] = (sc[j] & 0x3F) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (mn[j] & 0x3F) | ((mn[j + 4] >> 4) << 6)
        # bytes 8..11: low nibble = low four bits of scale j+4, high nibble = of min j+4
        s[j + 8] = (sc[j + 4] & 0x0F) | ((mn[j + 4] & 0x0F) << 4)
    return bytes(s)


def pack_quants(q: Sequence[int]) -> bytes:
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 16 for v in q)
    out = bytearray(128)
    for g in range(4):
        for l in range(32):
            out[32 * g + l] = q[64 * g + l] | (q[64 * g + 32 + l] << 4)
    return bytes(out)


def f16_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float16).view(np.uint16)[0])


def pack_block(d_bits: int, dmin_bits: int, sc, mn, q) -> bytes:
    hdr = bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF, dmin_bits & 0xFF, (dmin_bits >> 8) & 0xFF])
    blk = hdr + pack_scales_mins(sc, mn) + pack_quants(q)
    assert len(blk) == 144
    return blk


def pack_matrix(blocks_per_row: Sequence[Sequence[bytes]]) -> np.ndarray:
    rows = [b"".join(r) for r in blocks_per_row]
    return np.frombuffer(b"".join(rows), dtype=np.uint8).reshape(len(rows), -1).copy()

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


# ---------------------------------------------------------------- Q5_K, Q6_K
# Packers for the other two k-quant formats, written from the GGUF layout
# statements (independently of the oracle's decoders).

def pack_q5k_block(d_bits: int, dmin_bits: int, sc, mn, q) -> bytes:
    """176 bytes: d, dmin, the 12 scale/min bytes of Q4_K, 32 bytes whose bit
    j of byte l is the fifth bit of weight 32 j + l, then the low four bits
    of every weight packed as in Q4_K."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 32 for v in q)
    qh = bytearray(32)
    for j in range(8):
        for l in range(32):
            qh[l] |= ((q[32 * j + l] >> 4) & 1) << j
    hdr = bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF, dmin_bits & 0xFF, (dmin_bits >> 8) & 0xFF])
    blk = hdr + pack_scales_mins(sc, mn) + bytes(qh) + pack_quants([v & 15 for v in q])
    assert len(blk) == 176
    return blk


def pack_q6k_block(d_bits: int, scales, q) -> bytes:
    """210 bytes: 128 nibble bytes, 64 high-part bytes, 16 signed scales,
    fp16 d. Each half of 128 weights owns 64 nibble bytes and 32 high-part
    bytes: for l < 32, nibble byte l holds weights l (low) and 64 + l
    (high), nibble byte 32 + l holds 32 + l (low) and 96 + l (high), and
    high-part byte l holds the top two bits of weights l, 32 + l, 64 + l,
    96 + l in bits 0-1, 2-3, 4-5, 6-7."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 64 for v in q)
    scales = [int(v) for v in scales]
    assert len(scales) == 16 and all(-128 <= v < 128 for v in scales)
    ql = bytearray(128)
    qh = bytearray(64)
    for h in range(2):
        w = q[128 * h:128 * h + 128]
        for l in range(32):
            ql[64 * h + l] = (w[l] & 15) | ((w[64 + l] & 15) << 4)
            ql[64 * h + 32 + l] = (w[32 + l] & 15) | ((w[96 + l] & 15) << 4)
            qh[32 * h + l] = (w[l] >> 4) | ((w[32 + l] >> 4) << 2) | ((w[64 + l] >> 4) << 4) | ((w[96 + l] >> 4) << 6)
    sc = bytes([v & 0xFF for v in scales])
    blk = bytes(ql) + bytes(qh) + sc + bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF])
    assert len(blk) == 210
    return blk

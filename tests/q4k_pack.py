"""Test-side Q4_K encoder: builds super-blocks with chosen fields.

Used by tests to make structured inputs (constant quants, chosen scales,
subnormal d) for both the oracle and the HIP path.  It is written as the
*encoding* of the format reading (the inverse direction of a decoder) and is
pinned two ways: round trips through the oracle's decoder, and hand-packed
literal blocks in ``tests/golden/hand_blocks.txt`` that bypass it.

Format reading (the pages print no layout): fp16 d at byte 0, fp16 dmin at 2,
12 bytes of packed 6-bit scales/mins at 4, 128 quant bytes at 16.  Scale bytes:
bytes 0..3 carry sc[0..3] in their low 6 bits and the top 2 bits of sc[4..7];
bytes 4..7 carry mn[0..3] and the top 2 bits of mn[4..7]; bytes 8..11 carry the
low nibbles of sc[4..7] (low half) and of mn[4..7] (high half).  Quant byte
32g + r holds weight 64g + r in its low nibble and weight 64g + 32 + r in its
high nibble.
"""
from __future__ import annotations

import numpy as np


def pack_scales(sc, mn) -> np.ndarray:
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    assert len(sc) == 8 and len(mn) == 8
    assert all(0 <= v < 64 for v in sc + mn)
    s = np.zeros(12, np.uint8)
    for j in range(4):
        s[j] = (sc[j] & 0x3F) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (mn[j] & 0x3F) | ((mn[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 0x0F) | ((mn[j + 4] & 0x0F) << 4)
    return s


def pack_quants(q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64).reshape(256)
    assert q.min() >= 0 and q.max() < 16
    qs = np.zeros(128, np.uint8)
    for g in range(4):
        lo = q[64 * g: 64 * g + 32]
        hi = q[64 * g + 32: 64 * g + 64]
        qs[32 * g: 32 * g + 32] = (lo | (hi << 4)).astype(np.uint8)
    return qs


def f16_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float16).view(np.uint16)[0])


def pack_block(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    blk = np.zeros(144, np.uint8)
    blk[0] = d_bits & 0xFF
    blk[1] = (d_bits >> 8) & 0xFF
    blk[2] = dmin_bits & 0xFF
    blk[3] = (dmin_bits >> 8) & 0xFF
    blk[4:16] = pack_scales(sc, mn)
    blk[16:] = pack_quants(q)
    return blk


def random_fields(g: np.random.Generator):
    """Random (d_bits, dmin_bits, sc, mn, q) with the workload's distributions."""
    d = f16_bits(abs(g.standard_normal()) * 0.01)
    dmin = f16_bits(abs(g.standard_normal()) * 0.01)
    sc = g.integers(0, 64, 8)
    mn = g.integers(0, 64, 8)
    q = g.integers(0, 16, 256)
    return d, dmin, sc, mn, q

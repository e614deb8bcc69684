"""Test-side Q5_K encoder: builds super-blocks with chosen fields.

The encoding direction of the Q5_K format reading (GGUF convention; the pages
print no layout): the Q4_K super-block with 32 high-bit bytes between the
scales and the nibbles -- fp16 d at 0, fp16 dmin at 2, 12 scale bytes at 4,
qh[32] at 16, qs[128] at 48.  Weight 64g + r takes its low four bits from the
Q4_K nibble map and its fifth bit from bit 2g (r < 32) or 2g + 1 (r >= 32) of
qh[r mod 32].  Pinned by round trips through the oracle's decoder, by the
hand-packed literal blocks in ``tests/golden/hand_blocks_q5k.txt`` and by the
Q4_K cross-check (all high bits clear).
"""
from __future__ import annotations

import numpy as np

from q4k_pack import pack_quants, pack_scales


def pack_high_bits(q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64).reshape(256)
    assert q.min() >= 0 and q.max() < 32
    qh = np.zeros(32, np.uint8)
    for i in range(256):
        if q[i] >= 16:
            g, r = divmod(i, 64)
            qh[r % 32] |= 1 << (2 * g + (1 if r >= 32 else 0))
    return qh


def pack_q5k_block(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64).reshape(256)
    blk = np.zeros(176, np.uint8)
    blk[0] = d_bits & 0xFF
    blk[1] = (d_bits >> 8) & 0xFF
    blk[2] = dmin_bits & 0xFF
    blk[3] = (dmin_bits >> 8) & 0xFF
    blk[4:16] = pack_scales(sc, mn)
    blk[16:48] = pack_high_bits(q)
    blk[48:] = pack_quants(q % 16)
    return blk

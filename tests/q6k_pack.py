"""Test-side Q6_K encoder: builds blocks with chosen fields.

The encoding direction of the Q6_K format reading (GGUF convention; the pages
print no layout): ql[128] at 0, qh[64] at 128, signed 8-bit scales sc[16] at
192, fp16 d at 208.  Weight 128h + 32j + l keeps its low four bits in the low
(j < 2) or high (j >= 2) nibble of ql[64h + 32 (j mod 2) + l] and its top two
bits in bits 2j, 2j+1 of qh[32h + l].  Pinned by round trips through the
oracle's decoder and by the hand-packed literal blocks in
``tests/golden/hand_blocks_q6k.txt``.
"""
from __future__ import annotations

import numpy as np


def pack_q6k_block(d_bits: int, sc, q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64).reshape(256)
    sc = np.asarray(sc, dtype=np.int64).reshape(16)
    assert q.min() >= 0 and q.max() < 64 and sc.min() >= -128 and sc.max() < 128
    blk = np.zeros(210, np.uint8)
    for i in range(256):
        h, rem = divmod(i, 128)
        j, l = divmod(rem, 32)
        lo = 64 * h + 32 * (j % 2) + l
        blk[lo] |= (q[i] & 15) << (4 if j >= 2 else 0)
        blk[128 + 32 * h + l] |= (q[i] >> 4) << (2 * j)
    blk[192:208] = (sc & 0xFF).astype(np.uint8)
    blk[208] = d_bits & 0xFF
    blk[209] = (d_bits >> 8) & 0xFF
    return blk

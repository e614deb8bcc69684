"""Test-side Q3_K encoder: builds blocks with chosen fields.

The encoding direction of the Q3_K format reading (GGUF convention; the pages
print no layout): hmask[32] at 0, qs[64] at 32, 12 packed scale bytes at 96,
fp16 d at 108.  Weight 128h + 32j + l stores q + 4 (0..7): its low two bits in
bits 2j, 2j+1 of qs[32h + l], its third bit in bit 4h + j of hmask[l].
Sub-block t stores sc_t + 32 (0..63): the low nibble in s[t] (t < 8) or the
high nibble of s[t - 8], the top two bits in bits 2(t/4), 2(t/4)+1 of
s[8 + t mod 4].  Pinned by round trips through the oracle's decoder and by the
hand-packed blocks in ``tests/golden/hand_blocks_q3k.txt``.
"""
from __future__ import annotations

import numpy as np


def pack_q3k_block(d_bits: int, sc, q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64).reshape(256)
    sc = np.asarray(sc, dtype=np.int64).reshape(16)
    assert q.min() >= -4 and q.max() <= 3 and sc.min() >= -32 and sc.max() <= 31
    blk = np.zeros(110, np.uint8)
    for i in range(256):
        h, rem = divmod(i, 128)
        j, l = divmod(rem, 32)
        v = int(q[i]) + 4
        blk[32 + 32 * h + l] |= (v & 3) << (2 * j)
        blk[l] |= (v >> 2) << (4 * h + j)
    for t in range(16):
        u = int(sc[t]) + 32
        if t < 8:
            blk[96 + t] |= u & 15
        else:
            blk[96 + t - 8] |= (u & 15) << 4
        blk[96 + 8 + t % 4] |= (u >> 4) << (2 * (t // 4))
    blk[108] = d_bits & 0xFF
    blk[109] = (d_bits >> 8) & 0xFF
    return blk

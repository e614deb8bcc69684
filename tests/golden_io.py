"""Reader for the hand-packed block fixtures in tests/golden/."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expand(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            b, n = t.split("*")
            out += [int(b, 16)] * int(n)
        else:
            out.append(int(t, 16))
    return out


def hand_blocks(name: str = "hand_blocks.txt", block_bytes: int = 144):
    """Return {block name: (bytes uint8[block_bytes], expected fp64[256])}."""
    blocks = {}
    cur = None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            head, *rest = line.split()
            if head == "block":
                cur = rest[0]
                blocks[cur] = [None, None]
            elif head == "bytes":
                b = np.array(_expand(rest), dtype=np.uint8)
                assert b.size == block_bytes, (cur, b.size)
                blocks[cur][0] = b
            elif head == "expect":
                kind, *vals = rest
                e = np.zeros(256, np.float64)
                if kind == "subblock":
                    assert len(vals) == 8
                    for j, v in enumerate(vals):
                        e[32 * j: 32 * j + 32] = float(v)
                elif kind == "sparse":
                    for item in vals:
                        i, v = item.split(":")
                        e[int(i)] = float(v)
                elif kind == "rows":
                    for item in vals:
                        span, v = item.split(":")
                        i0, i1 = (int(t) for t in span.split("-"))
                        e[i0: i1 + 1] = float(v)
                else:
                    raise ValueError(kind)
                blocks[cur][1] = e
    return {k: (v[0], v[1]) for k, v in blocks.items()}

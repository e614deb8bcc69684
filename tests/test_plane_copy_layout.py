"""Host-side check of the copy addressing of the Q6_K / Q3_K GEMM whose operands go
through LDS (k_gemm_planes_lds in k_planes.hip): the kernel's index formulas restated in
Python and run over every lane of every copy.

For each weight super-block a workgroup copies, per tile row, the 16-byte units from the
boundary at or below the record's start into LDS unit PITCH * row + unit (PITCH = U + 1),
clamping any unit past the 16-byte boundary at or above the record's end to the one before
it; rows past n repeat row n - 1.  The test checks, for ragged N, uneven K splits and the
re-read copies past the last super-block, that no copy reads outside the matrix (whose byte
size the launcher requires to be a multiple of 16) and that every record lands intact at
the LDS offset the tile fill reads, including the two bytes before it that an aligned
dword read may touch.
"""
from __future__ import annotations

import numpy as np
import pytest

TILE_ROWS = 128
COPY_WAVES = 8  # waves issuing the copies (every wave of the workgroup)


def plane_stage(fmt):
    bb = 210 if fmt == 6 else 110
    u = 14 if fmt == 6 else 8
    pitch = u + 1
    wc = (TILE_ROWS * pitch + 64 * COPY_WAVES - 1) // (64 * COPY_WAVES)
    return bb, u, pitch, wc


def splits_for(m, n, k):
    tiles = ((m + 127) // 128) * ((n + 127) // 128)
    nb = k // 256
    splits = 1
    while tiles * splits * 2 <= 256 and splits * 2 <= nb // 2:
        splits *= 2
    per = (nb + splits - 1) // splits
    return (nb + per - 1) // per, per


@pytest.mark.parametrize("fmt", [6, 3])
@pytest.mark.parametrize("m,n,k", [(130, 200, 512), (300, 136, 2048), (64, 128, 256),
                                   (1000, 264, 768), (33, 40, 4096)])
def test_weight_copies_stay_in_the_matrix_and_land_every_record(fmt, m, n, k):
    bb, u, pitch, wc = plane_stage(fmt)
    nb = k // 256
    total = n * nb * bb
    assert total % 16 == 0, "the launcher sends this shape to the tile kernel"
    wbytes = np.random.default_rng(fmt * 1000 + n).integers(0, 256, total, dtype=np.uint8)
    row_bytes = nb * bb
    splits, per = splits_for(m, n, k)
    ui = (64 * np.arange(wc * COPY_WAVES)[:, None] + np.arange(64)[None, :]).ravel()
    r = ui // pitch
    unit = ui - r * pitch
    for z in range(splits):
        sb0 = z * per
        nsb = min(nb, sb0 + per) - sb0
        if nsb <= 0:
            continue
        for n0 in range(0, n, TILE_ROWS):
            wsrc = np.minimum(n0 + r, n - 1) * row_bytes + sb0 * bb
            for s in range(nsb + 2):  # the ring re-reads the last super-block past the end
                sc = min(s, nsb - 1)
                rec = wsrc + sc * bb
                last = ((rec + bb + 15) & ~15) - 16
                a = np.minimum((rec & ~15) + 16 * unit, last)
                assert a.min() >= 0 and a.max() + 16 <= total
                if s >= nsb:
                    continue
                lds = np.zeros(16 * ui.size, np.uint8)
                for lane_unit, src in zip(ui, a):
                    lds[16 * lane_unit:16 * lane_unit + 16] = wbytes[src:src + 16]
                for f_row in range(TILE_ROWS):
                    start = min(n0 + f_row, n - 1) * row_bytes + sb0 * bb
                    off = ((start & 15) + s * bb) & 15
                    rec0 = start + s * bb
                    p = f_row * pitch * 16 + off
                    assert p + bb <= f_row * pitch * 16 + u * 16
                    assert off % 4 != 2 or p - 2 >= f_row * pitch * 16
                    assert np.array_equal(lds[p:p + bb], wbytes[rec0:rec0 + bb])


@pytest.mark.parametrize("m,k", [(130, 512), (33, 4096), (1000, 768)])
def test_x_copies_stay_in_x(m, k):
    nb = k // 256
    splits, per = splits_for(m, 128, k)
    for z in range(splits):
        sb0 = z * per
        nsb = min(nb, sb0 + per) - sb0
        if nsb <= 0:
            continue
        nst = 4 * nsb
        for s in range(nst + 2):
            sc = min(s, nst - 1)
            # last element a lane's 16-byte copy reads: row m - 1, chunk 7
            e = (m - 1) * k + 256 * sb0 + 64 * sc + 8 * 7 + 8
            assert e <= m * k

"""Host-side bounds check of the GEMM's global -> LDS copy addressing (CPU
only; no kernel runs).

The copies of csrc/gemm_sr.hip are buffer loads to LDS: a buffer resource
whose base is the output tile's first row at K tile kt (A + m0*lda + kt*BK
elements, likewise for B), with 2**31 records, and a 32-bit lane offset
(clamped row * ld + chunk * 8) * 2 bytes, where the row is clamped to the
last row of the operand and the 16-byte chunk index c is the XOR swizzle of
the lane's chunk; chunks at or past K in the last K tile take the offset
2**31, which the hardware answers with zeros without touching memory. This
test restates that arithmetic for every tile configuration of the library
(256 x 256 with 64-deep K tiles, 128 x 128 in 4 and 8 waves, 64 x 64) and
checks, for every tile, copying wave, slab and lane, that each offset either
is the out-of-range value or addresses an element inside the operand's
first K columns of a valid row -- at the benchmark's 8192 x 14336 x 4096
and at ragged shapes."""

import numpy as np
import pytest

CONFIGS = {  # BM, BN, WM, WN, BK, STAGES, as in the library's tile configurations
    "big": (256, 256, 128, 64, 64, 2),
    "small": (128, 128, 64, 64, 64, 2),
    "small8": (128, 128, 64, 32, 64, 3),
    "tiny": (64, 64, 32, 32, 64, 4),
}
OUT_OF_RANGE = 1 << 31


def _offsets(cfg, m, n, k, lda, ldb):
    bm, bn, wm, wn, bk, _ = cfg
    waves = (bm // wm) * (bn // wn)
    row_bytes = bk * 2
    chunks = bk // 8
    slab_rows = 1024 // row_bytes
    slabs = (bm + bn) // slab_rows
    copiers = min(waves, 4)
    per_wave = slabs // copiers
    slabs_a = bm // slab_rows // copiers
    tiles_m, tiles_n = -(-m // bm), -(-n // bn)
    tm, tn = np.meshgrid(np.arange(tiles_m), np.arange(tiles_n), indexing="ij")
    tm, tn = tm.reshape(-1, 1, 1, 1), tn.reshape(-1, 1, 1, 1)
    wave = np.arange(copiers).reshape(1, -1, 1, 1)
    j = np.arange(per_wave).reshape(1, 1, -1, 1)
    lane = np.arange(64).reshape(1, 1, 1, -1)
    row = (wave + j * copiers) * slab_rows + lane // chunks
    if bk == 64:
        c = (lane % chunks) ^ ((row >> 1) & 7)
    else:
        c = (lane % chunks) ^ ((row >> 2) & 3)
    m0, n0 = tm * bm, tn * bn
    in_a = j < slabs_a
    rel = np.where(in_a, np.minimum(row, m - 1 - m0), np.minimum(row - bm, n - 1 - n0))
    ld = np.where(in_a, lda, ldb)
    voff = (rel * ld + c * 8) * 2
    return dict(in_a=np.broadcast_to(in_a, voff.shape), origin=np.where(in_a, m0, n0),
                rel=rel, c=c, voff=voff, ktiles=-(-k // bk), bk=bk, row_bytes=row_bytes)


@pytest.mark.parametrize("cfg", list(CONFIGS))
@pytest.mark.parametrize("shape", [(8192, 14336, 4096), (4100, 4097, 136), (33, 65, 72),
                                   (1, 1, 8), (300, 4105, 200)])
def test_copy_offsets_stay_inside_the_operands(cfg, shape):
    m, n, k = shape
    lda, ldb = k + 8 * (shape[0] % 3), k          # a padded and a tight leading dimension
    o = _offsets(CONFIGS[cfg], m, n, k, lda, ldb)
    voff, rel, c, bk = o["voff"], o["rel"], o["c"], o["bk"]
    # the offsets fit the resource's 2**31 records, and so the 32-bit argument
    assert voff.max() < OUT_OF_RANGE and voff.min() >= 0
    rows = np.where(o["in_a"], m, n)
    assert np.all(o["origin"] + rel <= rows - 1) and np.all(o["origin"] + rel >= 0)
    for kt in sorted({0, k // bk - 1, o["ktiles"] - 1} - {-1}):
        col = kt * bk + c * 8
        whole_tile = (kt + 1) * bk <= k
        # byte address relative to the operand's start, and the end of its
        # last valid row's first K columns
        ld = np.where(o["in_a"], lda, ldb)
        addr = (o["origin"] * ld + kt * bk) * 2 + voff
        last = ((rows - 1) * ld + k) * 2
        col, addr, last = np.broadcast_arrays(col, addr, last)
        live = np.ones(col.shape, dtype=bool) if whole_tile else col < k   # others read zeros
        # every live chunk's 8 elements lie in the row's first K columns
        assert np.all(col[live] + 8 <= k)
        assert np.all(addr[live] + 16 <= last[live])


@pytest.mark.parametrize("cfg", list(CONFIGS))
def test_copy_destinations_stay_inside_the_lds_ring(cfg):
    """Each wave-wide copy fills 1 KiB of LDS at stage * stage_bytes +
    slab * 1024; every stage's slabs tile that stage exactly, and the ring
    fits the 160 KiB of a CU."""
    bm, bn, wm, wn, bk, stages = CONFIGS[cfg]
    waves = (bm // wm) * (bn // wn)
    copiers = min(waves, 4)
    slabs = (bm + bn) * bk * 2 // 1024
    stage_bytes = (bm + bn) * bk * 2
    starts = sorted(s * stage_bytes + (w + j * copiers) * 1024
                    for s in range(stages) for w in range(copiers)
                    for j in range(slabs // copiers))
    assert slabs % copiers == 0
    assert starts == list(range(0, stages * stage_bytes, 1024))
    assert stages * stage_bytes <= 160 * 1024

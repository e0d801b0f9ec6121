"""Index math of the K/V tile layout in LDS (CPU).

The forward tile kernels (`tile_kernel` for d = 64, 128, 256 and the d = 64
HSTU split kernel) fill each K/V stage with direct HBM->LDS loads: wave
instruction i of wave w writes LDS bytes (w + 4 i) KB .. +1 KB of a tensor's
tile, lane l at byte offset 16 l, so each row of D bf16 (2 D bytes) is stored
unpadded, and the 16-byte chunk at LDS position (row r, chunk pc) holds the
tensor's chunk pc ^ kswz(r) (K) or pc ^ vswz(r) (V) of row r:

* kswz(r) = (r >> 1) & 7 for d = 64, r & 15 otherwise;
* vswz(r) = (r & 3) << 2 for d >= 128, (r & 2) << 1 for d = 64.

The kernels rely on three facts, checked here by enumeration for every tile
shape they use:

1. the loads of one tile write every 16-byte chunk of the tile exactly once
   and read every chunk of the tensor's rows exactly once (the swizzle is a
   bijection within each row);
2. a K fragment read (ds_read_b128; lane l reads row 32 kb + key_perm(l % 32),
   logical chunk 2 c + l // 32) puts the 16 lanes of each quarter-wave on 16
   distinct 16-byte bank groups of the 256-byte bank row, so it has no bank
   conflicts;
3. a V^T transposing read (ds_read_b64_tr_b16; lane l reads 8 bytes of row
   16 jj + 8 (l // 32) + (l % 16) // 4, logical chunk 4 db + 2 ((l >> 4) & 1) +
   (l & 3) // 2, byte 8 (l & 1) of it, and the same 4 rows further) touches,
   for each half-wave, 32 distinct 8-byte bank pairs.

The GPU parity tests check the kernels themselves; the counters show no LDS
bank conflicts for the bf16 kernels (profiles/).
"""

import itertools

import pytest


def kswz(r, d):
    return ((r >> 1) & 7) if d == 64 else (r & 15)


def vswz(r, d):
    return ((r & 3) << 2) if d >= 128 else ((r & 2) << 1)


def key_perm(m):
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1)


# (d, keys per tile) of the tile kernels: d = 128 and 256 use 32-key tiles, d = 64 64-key
# tiles; the d = 64 HSTU kernel loads 32-key tiles as four 1 KB pieces, one per wave
SHAPES = [(128, 32), (64, 64), (256, 32), (64, 32)]


@pytest.mark.parametrize("d,bn", SHAPES)
@pytest.mark.parametrize("which", ["k", "v"])
def test_direct_loads_cover_the_tile_once(d, bn, which):
    row_bytes = 2 * d
    tile = bn * row_bytes
    pieces = tile // 1024
    assert pieces % 4 == 0 or pieces == 4
    swz = kswz if which == "k" else vswz
    lds_chunks, src_chunks = [], []
    for piece in range(pieces):  # piece = w + 4 i
        for lane in range(64):
            byte = piece * 1024 + 16 * lane
            r, pc = byte // row_bytes, (byte % row_bytes) // 16
            lds_chunks.append((r, pc))
            src_chunks.append((r, pc ^ swz(r, d)))
    every = {(r, c) for r in range(bn) for c in range(row_bytes // 16)}
    assert len(lds_chunks) == len(every) and set(lds_chunks) == every
    assert len(src_chunks) == len(every) and set(src_chunks) == every


@pytest.mark.parametrize("d,bn", SHAPES)
def test_k_fragment_reads_have_no_bank_conflicts(d, bn):
    row_bytes = 2 * d
    for kb, c in itertools.product(range(bn // 32), range(d // 16)):
        for quarter in range(4):
            groups = []
            for lane in range(16 * quarter, 16 * quarter + 16):
                r = 32 * kb + key_perm(lane % 32)
                ch = (2 * c + lane // 32) ^ kswz(r, d)
                addr = r * row_bytes + 16 * ch
                groups.append((addr % 256) // 16)
            assert len(set(groups)) == 16, (d, bn, kb, c, quarter, groups)


@pytest.mark.parametrize("d,bn", SHAPES)
def test_v_transposing_reads_have_no_bank_conflicts(d, bn):
    row_bytes = 2 * d
    for kb, jj, db in itertools.product(range(bn // 32), range(2), range(d // 32)):
        for second in (0, 4):  # the read of rows 0..3 and the one of rows 4..7 of the 8-key group
            for half in range(2):
                pairs = []
                for lane in range(32 * half, 32 * half + 32):
                    tr_row = (lane & 15) >> 2
                    tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
                    tr_byte = 8 * (lane & 1)
                    krow = 32 * kb + 16 * jj + 8 * (lane >> 5) + tr_row + second
                    ch = (4 * db + tr_chunk) ^ vswz(krow - second, d)
                    # the kernels take the swizzle of the first row for both reads: rows
                    # krow and krow + 4 share it (vswz depends on the row's low two bits)
                    assert vswz(krow, d) == vswz(krow - second, d)
                    addr = krow * row_bytes + 16 * ch + tr_byte
                    pairs.append((addr % 256) // 8)
                assert len(set(pairs)) == 32, (d, bn, kb, jj, db, second, half)


def test_swizzles_permute_the_chunks_of_every_row():
    for d in (64, 128, 256):
        n = 2 * d // 16
        for r in range(64):
            assert sorted(c ^ kswz(r, d) for c in range(n)) == list(range(n))
            assert sorted(c ^ vswz(r, d) for c in range(n)) == list(range(n))

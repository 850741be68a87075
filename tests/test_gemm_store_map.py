"""Host-side model of where the projection GEMM's epilogue stores, and what
it reads as the residual (C = R + A . W^T, with C == R allowed in place);
and of the LDS transpose the kernel without a residual stores through.

The model follows the two-wave kernel's epilogue: 256 x 256 tiles, wave w
owns the 128 x 64 sub-tile (w & 1, w >> 1); lane l of a wave holds row
(w & 1) * 128 + 32 i + l % 32 of the tile (i = 0..3) and, per 32-column
block j and half gp, a 16-byte piece of 8 columns starting at
(w >> 1) * 64 + 32 j + 16 gp + 8 (l // 32).  Pieces go through a buffer
resource that ends at the tile's last row below M: the hardware drops a
store (and zeroes a load) at or past that end.

Checked: every element of rows < M is stored exactly once, by the lane that
read its residual at the same address; nothing is stored for rows >= M.
The superseded scheme (rows >= M clamped to M - 1, stores unmasked) is
modelled beside it to show the hazard the resource removes: other waves
then store row M - 1 as well, after reading it as their residual.
"""
import numpy as np
import pytest

BM = BN = 256


def lane_pieces(m0, n0, nc):
    """(wave, lane, row, first column, byte offset from the tile origin) of
    every piece of one tile."""
    out = []
    for w in range(8):
        wm, wn = w & 1, w >> 1
        for lane in range(64):
            for i in range(4):
                r = wm * 128 + i * 32 + lane % 32
                for j in range(2):
                    for gp in range(2):
                        c = wn * 64 + j * 32 + gp * 16 + (lane // 32) * 8
                        out.append((w, lane, m0 + r, n0 + c, (r * nc + c) * 2))
    return out


def stored_pieces(M, nc, clamp_old=False):
    """{(row, col): [(wave, lane, residual row)]} over all tiles."""
    hits = {}
    for m0 in range(0, M, BM):
        for n0 in range(0, nc, BN):
            tile_bytes = (min(M - m0, BM) * nc - n0) * 2
            for w, lane, row, col, off in lane_pieces(m0, n0, nc):
                if clamp_old:
                    row = min(row, M - 1)  # the old store address, unmasked
                elif off + 16 > tile_bytes:
                    assert row >= M, (row, col)
                    continue  # dropped by the range check
                hits.setdefault((row, col), []).append((w, lane, row))
    return hits


@pytest.mark.parametrize("M", [1, 15, 129, 255, 256, 300, 421, 17000, 55093 - 49152])
@pytest.mark.parametrize("nc", [256, 1024])
def test_each_valid_piece_stored_once_by_its_reader(M, nc):
    hits = stored_pieces(M, nc)
    assert set(hits) == {(r, c) for r in range(M) for c in range(0, nc, 8)}
    for (row, col), who in hits.items():
        assert len(who) == 1, (row, col, who)
        assert row < M and who[0][2] == row  # residual read at the stored row


@pytest.mark.parametrize("M", [15, 300, 55093 - 49152])
def test_old_clamp_let_other_waves_store_the_last_row(M):
    """With (M - 1) mod 256 < 128 the whole of wave group wm = 1 maps to row
    M - 1, so waves that do not own it read it as residual and store it."""
    assert (M - 1) % 256 < 128
    hits = stored_pieces(M, 256, clamp_old=True)
    last = [who for (row, _), who in hits.items() if row == M - 1]
    waves = {w for who in last for w, _, _ in who}
    assert any(len(who) > 1 for who in last)
    assert {w & 1 for w in waves} == {0, 1}


def transposed_pieces(m0, n0, nc):
    """Without a residual each wave writes its pieces into 8 KB of LDS, 64
    rows of 8 sixteen-byte chunks at a time (chunk c of row r at slot
    8 r + (c ^ (r mod 8))), and reads back slot-wise so that lane l of read
    s holds row s * 8 + l // 8, chunk l % 8: 8 lanes per 128-byte row.
    Returns (row, first column) stored per (wave, half, read, lane), after
    checking that each read gets the piece of the row and chunk it stores."""
    out = []
    for w in range(8):
        wm, wn = w & 1, w >> 1
        for h in range(2):
            slots = {}
            for ii in range(2):
                for j in range(2):
                    for gp in range(2):
                        for lane in range(64):
                            r = ii * 32 + lane % 32          # row within the half
                            c8 = j * 4 + gp * 2 + lane // 32  # piece column / 8
                            slot = r * 8 + (c8 ^ (r & 7))
                            assert slot not in slots
                            # the piece's true place in the MFMA layout
                            slots[slot] = (wm * 128 + (h * 2 + ii) * 32 + lane % 32,
                                           wn * 64 + j * 32 + gp * 16 + (lane // 32) * 8)
            assert sorted(slots) == list(range(512))
            for sread in range(8):
                for lane in range(64):
                    r = sread * 8 + lane // 8
                    c8 = lane % 8
                    row, col = wm * 128 + h * 64 + r, wn * 64 + c8 * 8
                    assert slots[r * 8 + (c8 ^ (r & 7))] == (row, col)
                    out.append((m0 + row, n0 + col, ((row * nc) + col) * 2))
    return out


@pytest.mark.parametrize("M", [15, 300, 55093 - 49152])
def test_transposed_stores_cover_each_valid_piece_once(M):
    nc = 512
    hits = {}
    for m0 in range(0, M, BM):
        for n0 in range(0, nc, BN):
            tile_bytes = (min(M - m0, BM) * nc - n0) * 2
            for row, col, off in transposed_pieces(m0, n0, nc):
                if off + 16 > tile_bytes:
                    assert row >= M
                    continue
                hits[(row, col)] = hits.get((row, col), 0) + 1
    assert hits == {(r, c): 1 for r in range(M) for c in range(0, nc, 8)}


def test_tile_bytes_fit_the_32_bit_resource():
    """The largest tile the API admits (Nc = 3 * 8192 for the projection)."""
    nc = 3 * 8192
    assert BM * nc * 2 < 2 ** 31
    offs = [off for *_, off in lane_pieces(0, nc - BN, nc)]
    assert max(offs) + 16 <= (BM * nc - (nc - BN)) * 2

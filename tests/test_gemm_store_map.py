"""Host-side model of where the projection GEMM's epilogue stores, and what
it reads as the residual (C = R + A . W^T, with C == R allowed in place);
and of the LDS transposes it stores through.

The model follows the two-wave kernel's epilogue: 256 x 256 tiles, wave w
owns the 128 x 64 sub-tile (w & 1, w >> 1); after the MFMA products lane l
of a wave holds row (w & 1) * 128 + 32 i + l % 32 of the tile (i = 0..3)
and, per 32-column block j and half gp, a 16-byte piece of 8 columns
starting at (w >> 1) * 64 + 32 j + 16 gp + 8 (l // 32).  Each wave
transposes these through its own LDS area, so that access s of lane l
covers row 8 s + l // 8 of the wave's rows, columns 8 (l % 8) .. + 7: 8
lanes per 128-byte row.  Without a residual the rounded bf16 pieces go
through LDS 64 rows at a time; with one, the fp32 sums go 32 rows at a
time, and the residual is loaded at the very address its sum is stored to.
Pieces go through a buffer resource that ends at the tile's last row below
M: the hardware drops a store (and zeroes a load) at or past that end.

Checked: every element of rows < M is stored exactly once, by the lane that
read its residual at the same address; nothing is stored for rows >= M;
each transpose hands every lane the sums of the row and columns it stores;
and the 16 lanes of each access of the fp32 transpose (a 256-byte window of
banks) touch 16 distinct 16-byte slots.  The superseded scheme (rows >= M clamped to
M - 1, stores unmasked) is modelled beside it to show the hazard the
resource removes: other waves then store row M - 1 as well, after reading
it as their residual.
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


def row_pieces(m0, n0, nc):
    """(wave, lane, row, first column, byte offset from the tile origin) of
    every whole-row access of one tile: access k of lane l covers row
    8 k + l // 8 of the wave's 128 rows (k = 0..15)."""
    out = []
    for w in range(8):
        wm, wn = w & 1, w >> 1
        for lane in range(64):
            for k in range(16):
                r = wm * 128 + 8 * k + lane // 8
                c = wn * 64 + 8 * (lane % 8)
                out.append((w, lane, m0 + r, n0 + c, (r * nc + c) * 2))
    return out


def stored_pieces(M, nc, clamp_old=False):
    """{(row, col): [(wave, lane, residual row)]} over all tiles: the
    residual is read by the same access that stores the sum (or, for the
    superseded scheme, the piece layout with rows clamped to M - 1)."""
    hits = {}
    for m0 in range(0, M, BM):
        for n0 in range(0, nc, BN):
            tile_bytes = (min(M - m0, BM) * nc - n0) * 2
            pieces = lane_pieces(m0, n0, nc) if clamp_old else row_pieces(m0, n0, nc)
            for w, lane, row, col, off in pieces:
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


def fp32_transposed_pieces(m0, n0, nc):
    """With a residual each wave writes its fp32 sums into 8 KB of LDS, 32
    rows of 16 four-column chunks at a time (chunk c of row r at slot
    16 r + (c ^ (r mod 16))), and reads back two chunks per lane so that
    lane l of read s holds row s * 8 + l // 8, columns 8 (l % 8) .. + 7.
    Returns (row, first column, byte offset) stored per (wave, quarter,
    read, lane), after checking that each read gets the sums of the row and
    columns it stores; the residual of access 4 i + s is loaded at the same
    offset."""
    out = []
    for w in range(8):
        wm, wn = w & 1, w >> 1
        for i in range(4):
            slots = {}
            for j in range(2):
                for gp in range(2):
                    for lane in range(64):
                        r = lane % 32
                        c = (j * 4 + gp * 2 + lane // 32) * 2
                        for t in range(2):  # columns 0..3, then 4..7 of the piece
                            slot = r * 16 + ((c + t) ^ (r & 15))
                            assert slot not in slots
                            slots[slot] = (wm * 128 + i * 32 + r,
                                           wn * 64 + j * 32 + gp * 16 + (lane // 32) * 8 + 4 * t)
            assert sorted(slots) == list(range(512))
            for sread in range(4):
                for lane in range(64):
                    r = sread * 8 + lane // 8
                    c = (lane % 8) * 2
                    row, col = wm * 128 + i * 32 + r, wn * 64 + (lane % 8) * 8
                    assert slots[r * 16 + (c ^ (r & 15))] == (row, col)
                    assert slots[r * 16 + ((c + 1) ^ (r & 15))] == (row, col + 4)
                    out.append((m0 + row, n0 + col, ((row * nc) + col) * 2))
    return out


@pytest.mark.parametrize("M", [15, 300, 55093 - 49152])
@pytest.mark.parametrize("transpose", [transposed_pieces, fp32_transposed_pieces])
def test_transposed_stores_cover_each_valid_piece_once(M, transpose):
    nc = 512
    hits = {}
    for m0 in range(0, M, BM):
        for n0 in range(0, nc, BN):
            tile_bytes = (min(M - m0, BM) * nc - n0) * 2
            for row, col, off in transpose(m0, n0, nc):
                if off + 16 > tile_bytes:
                    assert row >= M
                    continue
                hits[(row, col)] = hits.get((row, col), 0) + 1
    assert hits == {(r, c): 1 for r in range(M) for c in range(0, nc, 8)}


def _distinct_in_16_lane_groups(slot_of_lane):
    """The 16-byte slots of each group of 16 lanes fall on distinct 16-byte
    positions of a 256-byte window of banks."""
    for g0 in range(0, 64, 16):
        pos = {slot_of_lane(lane) % 16 for lane in range(g0, g0 + 16)}
        if len(pos) != 16:
            return False
    return True


def test_fp32_transpose_accesses_are_conflict_free():
    for j in range(2):
        for gp in range(2):
            for t in range(2):
                def wr(lane, j=j, gp=gp, t=t):
                    r, c = lane % 32, (j * 4 + gp * 2 + lane // 32) * 2 + t
                    return r * 16 + (c ^ (r & 15))
                assert _distinct_in_16_lane_groups(wr)
    for sread in range(4):
        for t in range(2):
            def rd(lane, sread=sread, t=t):
                r, c = sread * 8 + lane // 8, (lane % 8) * 2 + t
                return r * 16 + (c ^ (r & 15))
            assert _distinct_in_16_lane_groups(rd)


def test_tile_bytes_fit_the_32_bit_resource():
    """The largest tile the API admits (Nc = 3 * 8192 for the projection)."""
    nc = 3 * 8192
    assert BM * nc * 2 < 2 ** 31
    offs = [off for *_, off in lane_pieces(0, nc - BN, nc)]
    assert max(offs) + 16 <= (BM * nc - (nc - BN)) * 2

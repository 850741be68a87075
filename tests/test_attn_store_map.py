"""Host-side model of how the bf16 attention kernel writes a query tile's O
rows: 16 rows x 128 head columns (bf16) per tile, 64 lanes.

After the products and the pair swaps (v_permlane16_swap), lane (g4, l16),
lane = 16 g4 + l16, holds piece k = 0..3 of row l16: the 16-byte chunk
4 k + sg of the row's 16, with sg = (g4 mod 2) * 2 + g4 / 2.  Lanes l16 and
l16 ^ 8 of a group then trade one piece per half H (DPP row_ror:8, which
maps lane l16 of each 16-lane row to lane (l16 + 8) mod 16), and store
(H, b) writes, from lane (g4, l16), chunk 8 H + 4 (l16 / 8) + sg of row
(l16 mod 8) + 8 b.

Checked: every chunk of every valid row is written exactly once with the
data of that row and chunk; each store instruction covers 8 rows x 128
aligned bytes (8 lanes per row, consecutive chunks); rows past the item's
end are never written.
"""
import pytest


def native_pieces():
    """{(lane, k): (row, chunk)} after the pair swaps."""
    out = {}
    for lane in range(64):
        g4, l16 = lane >> 4, lane & 15
        sg = (g4 & 1) * 2 + (g4 >> 1)
        for k in range(4):
            out[(lane, k)] = (l16, 4 * k + sg)
    return out


def row_ror8(vals):
    """DPP row_ror:8 on a 64-lane register: lane i reads lane
    16 (i / 16) + (i + 8) mod 16."""
    return [vals[(i & ~15) | ((i + 8) & 15)] for i in range(64)]


def stores(nval):
    """[(H, b, [(lane, row, chunk, data)])] for one 16-row tile with nval
    valid rows; data is the (row, chunk) the lane's value came from."""
    have = native_pieces()
    out = []
    for H in range(2):
        send = [have[(lane, 2 * H if (lane & 15) >> 3 else 2 * H + 1)] for lane in range(64)]
        recv = row_ror8(send)
        for b in range(2):
            ins = []
            for lane in range(64):
                g4, l16 = lane >> 4, lane & 15
                hb, sg = l16 >> 3, (g4 & 1) * 2 + (g4 >> 1)
                v = have[(lane, 2 * H + b)] if hb == b else recv[lane]
                row = (l16 & 7) + 8 * b
                if row < nval:
                    ins.append((lane, row, 8 * H + 4 * hb + sg, v))
            out.append((H, b, ins))
    return out


@pytest.mark.parametrize("nval", [1, 7, 8, 9, 15, 16])
def test_each_chunk_once_with_its_own_data(nval):
    seen = {}
    for _, _, ins in stores(nval):
        for lane, row, chunk, data in ins:
            assert data == (row, chunk), (lane, row, chunk, data)
            seen[(row, chunk)] = seen.get((row, chunk), 0) + 1
    assert seen == {(r, c): 1 for r in range(nval) for c in range(16)}


def test_each_store_is_8_rows_of_128_bytes():
    for H, b, ins in stores(16):
        rows = {}
        for lane, row, chunk, _ in ins:
            rows.setdefault(row, []).append(chunk)
        assert len(rows) == 8 and len(ins) == 64
        for row, chunks in rows.items():
            assert sorted(chunks) == list(range(8 * H, 8 * H + 8))  # one aligned 128-byte half

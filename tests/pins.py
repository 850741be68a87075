"""Checks that pin the CPU oracle to facts other than itself.

Each `pin_*` takes an oracle handle and raises AssertionError on a mismatch.
They are collected by test_oracle_pins.py (against the real oracle) and by
test_oracle_mutants.py (against copies of the oracle with planted mistakes,
each of which at least one pin must reject).

What the sub-layer is (IBM model card, "Model Architecture" (1): block
attention over 4-second blocks in every conformer layer; usage section:
sequence packing with non-causal attention): per block of at most B rows,
restarting at every sequence, softmax(Q K^T / sqrt(dh)) V per head, then the
output projection plus the residual.

Independent references used here:
  * closed form for B = 1 (every block is one row, softmax weight 1):
    out = x + (x Wv^T) Wo^T
  * torch's scaled_dot_product_attention (CPU, float64) when one block covers
    a whole sequence
  * a brute-force masked full-attention computation in numpy
  * exact invariances (packing, block/sequence split, locality, zero weights,
    power-of-two rescaling, constant rows, uniform attention)
"""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_problem(lengths, d=32, heads=2, seed=0, wscale=None):
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    n = int(lengths.sum())
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    s = (1.0 / np.sqrt(d)) if wscale is None else wscale
    x = rng.standard_normal((n, d))
    wqkv = rng.standard_normal((3 * d, d)) * s
    wo = rng.standard_normal((d, d)) * s
    return x, cu, wqkv, wo


def brute_force(x, cu, wqkv, wo, block, heads):
    """Full N x N attention with a mask allowing only same-sequence, same-block pairs."""
    n, d = x.shape
    dh = d // heads
    qkv = x @ wqkv.T
    seq = np.zeros(n, np.int64)
    pos = np.zeros(n, np.int64)
    for s in range(len(cu) - 1):
        seq[cu[s]:cu[s + 1]] = s
        pos[cu[s]:cu[s + 1]] = np.arange(cu[s + 1] - cu[s])
    blk = pos // block
    allowed = (seq[:, None] == seq[None, :]) & (blk[:, None] == blk[None, :])
    o = np.zeros((n, d))
    for h in range(heads):
        q = qkv[:, h * dh:(h + 1) * dh]
        k = qkv[:, d + h * dh:d + (h + 1) * dh]
        v = qkv[:, 2 * d + h * dh:2 * d + (h + 1) * dh]
        z = (q @ k.T) / np.sqrt(dh)
        z = np.where(allowed, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)
        o[:, h * dh:(h + 1) * dh] = p @ v
    return x + o @ wo.T


def brute_force_padded(x, lengths, bucket, wqkv, wo, block, heads):
    """Padded buckets x [S*T, d] straight in the padded layout: full
    (S*T) x (S*T) attention where a query may see a key only if both are
    valid rows of the same bucket and the same block; padding rows get a
    zero attention output."""
    n, d = x.shape
    dh = d // heads
    qkv = x @ wqkv.T
    row = np.arange(n)
    bkt, pos = row // bucket, row % bucket
    valid = pos < np.clip(np.asarray(lengths), 0, bucket)[bkt]
    blk = pos // block
    allowed = ((bkt[:, None] == bkt[None, :]) & (blk[:, None] == blk[None, :]) &
               valid[:, None] & valid[None, :])
    o = np.zeros((n, d))
    for h in range(heads):
        q = qkv[:, h * dh:(h + 1) * dh]
        k = qkv[:, d + h * dh:d + (h + 1) * dh]
        v = qkv[:, 2 * d + h * dh:2 * d + (h + 1) * dh]
        z = np.where(allowed, (q @ k.T) / np.sqrt(dh), -np.inf)
        for i in np.nonzero(valid)[0]:
            zi = z[i] - z[i].max()
            p = np.exp(zi)
            o[i, h * dh:(h + 1) * dh] = (p / p.sum()) @ v
    return x + o @ wo.T


def rel_err(a, b):
    scale = np.sqrt(np.mean(np.square(b))) if b.size else 1.0
    return float(np.max(np.abs(a - b)) / max(scale, 1e-300)) if b.size else 0.0


# ---------------------------------------------------------------------------
# pins

def pin_block1_closed_form(orc):
    """B = 1: each row attends only to itself, so out = x + (x Wv^T) Wo^T."""
    x, cu, wqkv, wo = rand_problem([5, 3, 7], d=32, heads=4, seed=1)
    d = x.shape[1]
    ref = x + (x @ wqkv[2 * d:].T) @ wo.T
    got = orc.block_mhsa(x, cu, wqkv, wo, 1, 4)
    assert rel_err(got, ref) < 1e-13, rel_err(got, ref)


def pin_full_attention_sdpa(orc):
    """B >= every length: per-sequence full bidirectional attention (library routine)."""
    lengths = [9, 1, 17, 4]
    heads, d = 4, 32
    dh = d // heads
    x, cu, wqkv, wo = rand_problem(lengths, d=d, heads=heads, seed=2, wscale=0.4)
    got = orc.block_mhsa(x, cu, wqkv, wo, 1000, heads)
    xt = torch.from_numpy(x)
    W = torch.from_numpy(wqkv)
    ref = np.zeros_like(x)
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        xs = xt[a:b]
        q = (xs @ W[:d].T).reshape(b - a, heads, dh).transpose(0, 1)
        k = (xs @ W[d:2 * d].T).reshape(b - a, heads, dh).transpose(0, 1)
        v = (xs @ W[2 * d:].T).reshape(b - a, heads, dh).transpose(0, 1)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=False)
        o = o.transpose(0, 1).reshape(b - a, d).numpy()
        ref[a:b] = x[a:b] + o @ wo.T
    assert rel_err(got, ref) < 1e-12, rel_err(got, ref)


def pin_brute_force_mask(orc):
    """Blocks restart at each sequence; tails are partial (brute-force masked attention)."""
    cases = [([7, 3, 12, 1, 9], 4, 4), ([20], 6, 2), ([5, 5, 5], 2, 1), ([13, 2], 16, 4),
             ([11, 4, 9], 5, 2)]
    for i, (lengths, block, heads) in enumerate(cases):
        x, cu, wqkv, wo = rand_problem(lengths, d=32, heads=heads, seed=10 + i, wscale=0.35)
        got = orc.block_mhsa(x, cu, wqkv, wo, block, heads)
        ref = brute_force(x, cu, wqkv, wo, block, heads)
        assert rel_err(got, ref) < 1e-12, (lengths, block, heads, rel_err(got, ref))


def pin_packing_invariance(orc):
    """Packing sequences equals running them one at a time (bitwise)."""
    lengths = [6, 11, 3, 8]
    x, cu, wqkv, wo = rand_problem(lengths, d=32, heads=2, seed=3)
    packed = orc.block_mhsa(x, cu, wqkv, wo, 4, 2)
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        one = orc.block_mhsa(x[a:b], np.array([0, b - a], np.int32), wqkv, wo, 4, 2)
        assert np.array_equal(one, packed[a:b]), s


def pin_block_split(orc):
    """Cutting every sequence at its block boundaries and using B = inf gives the same bits."""
    lengths = [10, 7]
    B = 4
    x, cu, wqkv, wo = rand_problem(lengths, d=32, heads=2, seed=4)
    ref = orc.block_mhsa(x, cu, wqkv, wo, B, 2)
    pieces = []
    for ln in lengths:
        pieces += [min(B, ln - j) for j in range(0, ln, B)]
    cu2 = np.zeros(len(pieces) + 1, np.int32)
    cu2[1:] = np.cumsum(pieces)
    got = orc.block_mhsa(x, cu2, wqkv, wo, 10 ** 6, 2)
    assert np.array_equal(got, ref)


def pin_locality(orc):
    """Changing the rows of one block changes only that block's outputs."""
    x, cu, wqkv, wo = rand_problem([9, 6], d=32, heads=2, seed=5)
    B = 4  # blocks: [0,4) [4,8) [8,9) [9,13) [13,15)
    ref = orc.block_mhsa(x, cu, wqkv, wo, B, 2)
    x2 = x.copy()
    x2[4:8] += 0.5
    got = orc.block_mhsa(x2, cu, wqkv, wo, B, 2)
    keep = np.ones(len(x), bool)
    keep[4:8] = False
    assert np.array_equal(got[keep], ref[keep])
    assert np.all(np.abs(got[4:8] - ref[4:8]).max(axis=1) > 0)


def pin_zero_weights(orc):
    """Wo = 0 or Wv = 0 leaves out == x exactly."""
    x, cu, wqkv, wo = rand_problem([5, 9], d=32, heads=2, seed=6)
    d = x.shape[1]
    got = orc.block_mhsa(x, cu, wqkv, np.zeros_like(wo), 3, 2)
    assert np.array_equal(got, x)
    w = wqkv.copy()
    w[2 * d:] = 0
    got = orc.block_mhsa(x, cu, w, wo, 3, 2)
    assert np.array_equal(got, x)


def pin_power_of_two_qk(orc):
    """Scaling Wq by 2^k and Wk by 2^-k leaves every logit, hence the output, bit-identical."""
    x, cu, wqkv, wo = rand_problem([8, 5], d=32, heads=2, seed=7)
    d = x.shape[1]
    w = wqkv.copy()
    w[:d] *= 8.0
    w[d:2 * d] *= 0.125
    a = orc.block_mhsa(x, cu, wqkv, wo, 3, 2)
    b = orc.block_mhsa(x, cu, w, wo, 3, 2)
    assert np.array_equal(a, b)


def pin_permutation_within_block(orc):
    """Permuting rows inside one block permutes that block's outputs (bidirectional, no position)."""
    x, cu, wqkv, wo = rand_problem([10], d=32, heads=2, seed=8)
    ref = orc.block_mhsa(x, cu, wqkv, wo, 5, 2)
    perm = np.arange(10)
    perm[5:] = [8, 5, 9, 7, 6]
    got = orc.block_mhsa(x[perm], cu, wqkv, wo, 5, 2)
    assert rel_err(got, ref[perm]) < 1e-13


def pin_constant_rows(orc):
    """All rows of a block equal: every weight is 1/L, so out = x + v Wo^T for each row."""
    x, cu, wqkv, wo = rand_problem([6], d=32, heads=2, seed=9)
    d = x.shape[1]
    x[:] = x[0]
    got = orc.block_mhsa(x, cu, wqkv, wo, 6, 2)
    ref = x + (x @ wqkv[2 * d:].T) @ wo.T
    assert rel_err(got, ref) < 1e-13


def pin_uniform_attention(orc):
    """Wq = 0: all logits are 0, so each row gets the mean value row of its own block."""
    lengths = [9, 4, 7]
    B = 4
    x, cu, wqkv, wo = rand_problem(lengths, d=32, heads=2, seed=11)
    d = x.shape[1]
    w = wqkv.copy()
    w[:d] = 0
    got = orc.block_mhsa(x, cu, w, wo, B, 2)
    v = x @ wqkv[2 * d:].T
    mean_v = np.zeros_like(v)
    for s in range(len(lengths)):
        for a in range(int(cu[s]), int(cu[s + 1]), B):
            b = min(a + B, int(cu[s + 1]))
            mean_v[a:b] = v[a:b].mean(axis=0)
    ref = x + mean_v @ wo.T
    assert rel_err(got, ref) < 1e-13


def pin_empty_and_degenerate(orc):
    """Zero-length sequences produce no rows; all-empty packs are a no-op; B > N is full attention."""
    x, cu, wqkv, wo = rand_problem([0, 5, 0, 0, 3, 0], d=32, heads=2, seed=12)
    got = orc.block_mhsa(x, cu, wqkv, wo, 2, 2)
    ref = orc.block_mhsa(x, np.array([0, 5, 8], np.int32), wqkv, wo, 2, 2)
    assert np.array_equal(got, ref)
    empty = orc.block_mhsa(np.zeros((0, 32)), np.zeros(3, np.int32), wqkv, wo, 2, 2)
    assert empty.shape == (0, 32)


def pin_golden_block_tables(orc):
    """Block tables of the 8.43 s clip (422 frames) and the 800-frame bucket (cited fixtures)."""
    for name in ("block_table_t422.txt", "block_table_bucket800.txt"):
        rows, frames, block = [], None, None
        with open(os.path.join(GOLDEN, name)) as f:
            for line in f:
                line = line.split("#")[0].strip()
                if not line:
                    continue
                k, v = line.split()
                if k == "frames":
                    frames = int(v)
                elif k == "block_frames":
                    block = int(v)
                else:
                    rows.append((int(k), int(v)))
        st, ln = orc.block_table(np.array([0, frames], np.int32), block)
        assert list(zip(st.tolist(), ln.tolist())) == rows, name


def pin_row_mask(orc):
    """Computing selected rows only gives the same bits as the full computation."""
    x, cu, wqkv, wo = rand_problem([9, 6, 11], d=32, heads=2, seed=13)
    ref = orc.block_mhsa(x, cu, wqkv, wo, 4, 2)
    mask = np.zeros(len(x), np.uint8)
    mask[[0, 5, 10, 17, 25]] = 1
    got = orc.block_mhsa(x, cu, wqkv, wo, 4, 2, mask=mask)
    sel = mask.astype(bool)
    assert np.array_equal(got[sel], ref[sel])
    assert np.all(np.isnan(got[~sel]))


def pin_thread_invariance(orc):
    x, cu, wqkv, wo = rand_problem([13, 7, 9], d=32, heads=4, seed=14)
    a = orc.block_mhsa(x, cu, wqkv, wo, 5, 4, nthreads=1)
    b = orc.block_mhsa(x, cu, wqkv, wo, 5, 4, nthreads=7)
    assert np.array_equal(a, b)


def pin_stages_compose(orc):
    """The staged entry points compose to the whole sub-layer, bit for bit."""
    x, cu, wqkv, wo = rand_problem([7, 10], d=32, heads=2, seed=15)
    qkv = orc.qkv_proj(x, wqkv)
    o = orc.block_attn(qkv, cu, 2, 3)
    out = orc.out_proj_residual(o, wo, x)
    assert np.array_equal(out, orc.block_mhsa(x, cu, wqkv, wo, 3, 2))
    assert rel_err(qkv, x @ wqkv.T) < 1e-13


def pin_padded_buckets(orc):
    """Padded buckets against a masked brute force written in the padded
    layout (blocks restart in every bucket, padding is never a key); padding
    rows return x; what padding rows hold never reaches a valid row; lengths
    past the bucket are clamped to it."""
    rng = np.random.default_rng(11)
    lengths, t, block, heads, d = [7, 0, 12, 3], 12, 5, 2, 16
    n = len(lengths) * t
    x = rng.standard_normal((n, d))
    wqkv = rng.standard_normal((3 * d, d)) / 4
    wo = rng.standard_normal((d, d)) / 4
    got = orc.block_mhsa_padded(x, lengths, t, wqkv, wo, block, heads)
    ref = brute_force_padded(x, lengths, t, wqkv, wo, block, heads)
    assert rel_err(got, ref) < 1e-12
    pos = np.arange(n) % t
    pad = pos >= np.asarray(lengths)[np.arange(n) // t]
    assert np.array_equal(got[pad], x[pad])
    x2 = x.copy()
    x2[pad] = 1e3 * rng.standard_normal((int(pad.sum()), d))
    got2 = orc.block_mhsa_padded(x2, lengths, t, wqkv, wo, block, heads)
    assert np.array_equal(got2[~pad], got[~pad])
    assert np.array_equal(got2[pad], x2[pad])
    got3 = orc.block_mhsa_padded(x, [7, -4, 99, 3], t, wqkv, wo, block, heads)
    assert np.array_equal(got3, got)


def _xattn_problem(lengths, window, nq=3, f=24, dq=16, seed=0):
    rng = np.random.default_rng(seed)
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    from oracle import window_xattn as wx
    nw = wx.num_windows(cu, window)
    hcat = rng.standard_normal((int(cu[-1]), f))
    xq = rng.standard_normal((nw, nq, dq))
    wq = rng.standard_normal((dq, dq)) / 4
    wkv = rng.standard_normal((2 * dq, f)) / 5
    wo = rng.standard_normal((dq, dq)) / 4
    return cu, hcat, xq, wq, wkv, wo


def pin_window_xattn_brute_force(orc):
    """Window cross-attention against one masked attention over all frames:
    every query row of every window against every frame, with a mask that
    keeps only the frames of its own window."""
    from oracle import window_xattn as wx
    lengths, window, heads = [31, 15, 4, 0, 16], 15, 2
    cu, hcat, xq, wq, wkv, wo = _xattn_problem(lengths, window, seed=3)
    got = wx.window_xattn(hcat, cu, xq, wq, wkv, wo, heads, window)
    nw, nq, dq = xq.shape
    dh = dq // heads
    # window index of every frame, by walking the sequences frame by frame
    win_of = np.full(int(cu[-1]), -1)
    w = 0
    for s in range(len(lengths)):
        for j in range(lengths[s]):
            win_of[cu[s] + j] = w + j // window
        w += -(-lengths[s] // window)
    assert w == nw and (win_of >= 0).all()
    q = xq.reshape(nw * nq, dq) @ wq.T
    k = hcat @ wkv[:dq].T
    v = hcat @ wkv[dq:].T
    qwin = np.repeat(np.arange(nw), nq)
    allowed = qwin[:, None] == win_of[None, :]
    o = np.zeros((nw * nq, dq))
    for h in range(heads):
        c = slice(h * dh, (h + 1) * dh)
        z = np.where(allowed, (q[:, c] @ k[:, c].T) / np.sqrt(dh), -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        o[:, c] = (p / p.sum(axis=1, keepdims=True)) @ v[:, c]
    ref = (xq.reshape(nw * nq, dq) + o @ wo.T).reshape(nw, nq, dq)
    assert rel_err(got, ref) < 1e-12


def pin_window_xattn_closed_forms(orc):
    """A one-frame window gives every query that frame's value row (softmax
    weight 1): out = xq + (h Wv^T) Wo^T; Wo = 0 gives out = xq; frames
    permuted inside a window change nothing; the windows of a sequence do
    not see each other (changing one window's frames leaves the others)."""
    from oracle import window_xattn as wx
    cu, hcat, xq, wq, wkv, wo = _xattn_problem([1, 1, 3], 1, seed=4)
    dq = xq.shape[2]
    got = wx.window_xattn(hcat, cu, xq, wq, wkv, wo, 2, 1)
    ref = xq + ((hcat @ wkv[dq:].T) @ wo.T)[:, None, :]
    assert rel_err(got, ref) < 1e-13
    cu, hcat, xq, wq, wkv, wo = _xattn_problem([40, 7], 15, seed=5)
    z = wx.window_xattn(hcat, cu, xq, wq, wkv, np.zeros_like(wo), 2, 15)
    assert np.array_equal(z, xq)
    base = wx.window_xattn(hcat, cu, xq, wq, wkv, wo, 2, 15)
    perm = hcat.copy()
    perm[15:30] = perm[15:30][::-1]
    assert rel_err(wx.window_xattn(perm, cu, xq, wq, wkv, wo, 2, 15), base) < 1e-13
    other = hcat.copy()
    other[15:30] += 3.0
    moved = wx.window_xattn(other, cu, xq, wq, wkv, wo, 2, 15)
    assert np.array_equal(moved[[0, 2, 3]], base[[0, 2, 3]])
    assert not np.allclose(moved[1], base[1])


def read_ctc_golden(name="ctc_pool_small.txt"):
    """(classes, lengths, blank_prob, logits, argmax, tokens per sequence) of a fixture."""
    rows, argmax, tokens = [], None, {}
    classes = lengths = None
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("classes"):
            classes = int(line.split()[1])
        elif line.startswith("lengths"):
            lengths = [int(v) for v in line.split()[1:]]
        elif line.startswith("argmax"):
            argmax = [int(v) for v in line.split()[1:]]
        elif line.startswith("tokens"):
            k, v = line[len("tokens"):].split(":")
            tokens[int(k)] = [int(t) for t in v.split()]
        else:
            rows.append([float(v) for v in line.split()])
    rows = np.asarray(rows)
    assert rows.shape == (sum(lengths), classes + 1)
    return classes, lengths, rows[:, 0], rows[:, 1:], argmax, [tokens[i] for i in range(len(lengths))]


def pin_ctc_pool_golden(orc):
    """The hand-worked fixture: window 4, stride 2, weights 1 - blank
    probability, ties to the lowest class, merge, drop blanks, minus one."""
    from oracle import ctc_pool as cp
    classes, lengths, bp, logits, argmax, tokens = read_ctc_golden()
    cu = np.concatenate([[0], np.cumsum(lengths)])
    got = cp.pooled_argmax(logits, bp, cu)
    assert got.tolist() == argmax
    dec = cp.ctc_greedy(got, cp.positions(lengths))
    assert [t.tolist() for t in dec] == tokens


def pin_ctc_pool_constructed(orc):
    """Decoding recovers token sequences that the inputs were built from: each
    token becomes one or more pooled positions (repeats), with blanks between
    equal neighbours and at random; every frame pair of position j carries its
    class with a margin over noise, and pair weights halve along the sequence
    (1 - blank probability = 2^-j) so each pooled window is won by its first
    pair."""
    from oracle import ctc_pool as cp
    rng = np.random.default_rng(21)
    classes = 40
    want, logits, bp, lengths = [], [], [], []
    for _ in range(5):
        toks = rng.integers(0, classes - 1, size=int(rng.integers(0, 7)))
        seq = []  # winning class per position
        for i, t in enumerate(toks):
            if seq and (seq[-1] == t + 1 or rng.random() < 0.4):
                seq.append(0)
            seq += [int(t) + 1] * int(rng.integers(1, 3))
        seq += [0] * int(rng.integers(0, 2))
        if len(seq) > 24:
            continue
        n = 2 * len(seq) - int(rng.integers(0, 2)) if seq else 0  # odd lengths too
        for t in range(n):
            j = t // 2
            row = rng.uniform(-1, 1, classes)
            row[seq[j]] += 20.0
            logits.append(row)
            bp.append(1.0 - 2.0 ** -j)
        lengths.append(n)
        want.append([int(t) for t in toks])
    logits = np.asarray(logits, np.float32).reshape(-1, classes)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    ids = cp.pooled_argmax(logits, np.asarray(bp, np.float32), cu)
    got = cp.ctc_greedy(ids, cp.positions(lengths))
    assert [g.tolist() for g in got] == want, (got, want)


def pooled_scores_f64(logits, blank_prob, lengths, window=4, stride=2):
    """Pooled class scores in fp64 straight from the definition (model card,
    "Model Architecture" (1): windows of `window` frames weighted by
    1 - blank probability; stride 2 from the ONNX export's 211 positions for
    422 frames), and the fp32 rounding bound of each: a pooled score sums at
    most `window` products w_t * l_t with w_t = 1 - b_t, and the fp32 order
    rounds w_t, each product and each partial sum once, so
    |s32 - s64| <= g * sum_t |w_t l_t|, g = n u / (1 - n u), n = window + 2,
    u = 2^-24 (the forward error bound of a recursive sum).
    Returns (scores [P, C], bound [P, C])."""
    logits = np.asarray(logits, np.float64)
    w = 1.0 - np.asarray(blank_prob, np.float64)
    u = 2.0 ** -24
    n = window + 2
    g = n * u / (1 - n * u)
    scores, bounds = [], []
    first = 0
    for ln in lengths:
        for start in range(0, ln, stride):
            rows = np.arange(first + start, first + min(start + window, ln))
            terms = w[rows, None] * logits[rows]
            scores.append(terms.sum(axis=0))
            bounds.append(g * np.abs(terms).sum(axis=0))
        first += ln
    c = logits.shape[1]
    return (np.asarray(scores).reshape(-1, c), np.asarray(bounds).reshape(-1, c))


def decisive(scores, bounds):
    """Positions whose fp64 winner beats every other class by more than the
    two rounding bounds together (there, any order of fp32 rounding picks the
    same class), and the fp64 winners."""
    top = np.argmax(scores, axis=1)
    rows = np.arange(len(top))
    lead = scores[rows, top][:, None] - scores - (bounds[rows, top][:, None] + bounds)
    lead[rows, top] = np.inf
    return lead.min(axis=1) > 0, top


def pin_ctc_pool_fp64_margin(orc):
    """The oracle's fp32-order argmax equals the argmax of fp64 pooled scores
    computed from the definition wherever the fp64 lead exceeds the fp32
    rounding bound (and such positions are nearly all of them)."""
    from oracle import ctc_pool as cp
    rng = np.random.default_rng(31)
    lengths, classes = [41, 1, 0, 30, 2], 3000
    n = sum(lengths)
    logits = torch.from_numpy(rng.standard_normal((n, classes)).astype(np.float32)).to(
        torch.bfloat16).float().numpy()
    logits[:, 0] += 1.0
    bp = rng.uniform(0, 1, n).astype(np.float32)
    got = cp.pooled_argmax(logits, bp, np.concatenate([[0], np.cumsum(lengths)]))
    s64, bound = pooled_scores_f64(logits, bp, lengths)
    ok, top = decisive(s64, bound)
    assert len(got) == len(top) == int(cp.positions(lengths).sum())
    assert ok.mean() > 0.9
    assert np.array_equal(got[ok], top[ok])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

"""CPU oracle for the window cross-attention of the Q-Former projector.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product package never imports this.

What it computes (IBM model card, "Model Architecture" (2) Q-Former
Projector: a 2-layer window Q-Former reduces each 15-frame window of the
concatenated hidden states of encoder layers 4, 8, 12 and 16 to 3 queries by
cross-attention).  The pages give neither widths nor head count nor the
treatment of a sequence's last, shorter window; the readings used are:

  * windows: non-overlapping runs of `window` frames from each sequence's
    first frame; the last one holds the remainder and still yields `nq`
    query rows;
  * features hcat [N][F], F = 4 d (the four layers side by side);
  * query states xq [W][nq][dq], one set per window (the output of the
    Q-Former's self-attention; for its first layer the same learned queries
    in every window);
  * projections without bias: q = xq Wq^T, k | v = hcat Wkv^T (K rows then V
    rows of Wkv [2 dq][F]), heads of dh = dq / heads, logits scaled by
    1/sqrt(dh), softmax over the window's frames, out = xq + o Wo^T.

Everything is IEEE double; the projections and the per-window products are
numpy matrix products (a library primitive per step), the softmax is the
two-pass definition.  Pinned in tests/pins.py (brute force over a
window-masked full attention, a one-frame window's closed form, invariances).
"""
from __future__ import annotations

import numpy as np


def window_table(cu, window: int):
    """(first row, frames) of every window, sequence by sequence."""
    cu = np.asarray(cu, np.int64)
    rows, lens = [], []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for r in range(a, b, window):
            rows.append(r)
            lens.append(min(window, b - r))
    return np.asarray(rows, np.int64), np.asarray(lens, np.int64)


def num_windows(cu, window: int) -> int:
    return len(window_table(cu, window)[0])


def window_xattn(hcat, cu, xq, wq, wkv, wo, heads: int, window: int, windows=None):
    """out [W][nq][dq] (NaN for windows not listed in `windows`, if given)."""
    hcat = np.asarray(hcat, np.float64)
    xq = np.asarray(xq, np.float64)
    wq, wkv, wo = (np.asarray(w, np.float64) for w in (wq, wkv, wo))
    nw, nq, dq = xq.shape
    dh = dq // heads
    row0, lens = window_table(cu, window)
    if len(row0) != nw:
        raise ValueError(f"xq holds {nw} windows, the sequences make {len(row0)}")
    out = np.full(xq.shape, np.nan)
    todo = range(nw) if windows is None else sorted(set(int(w) for w in windows))
    wk, wv = wkv[:dq], wkv[dq:]
    for w in todo:
        h = hcat[row0[w]:row0[w] + lens[w]]          # [L, F]
        q = xq[w] @ wq.T                               # [nq, dq]
        k = h @ wk.T                                   # [L, dq]
        v = h @ wv.T
        o = np.zeros((nq, dq))
        for hd in range(heads):
            c = slice(hd * dh, (hd + 1) * dh)
            z = (q[:, c] @ k[:, c].T) / np.sqrt(dh)   # [nq, L]
            z = z - z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p /= p.sum(axis=1, keepdims=True)
            o[:, c] = p @ v[:, c]
        out[w] = xq[w] + o @ wo.T
    return out

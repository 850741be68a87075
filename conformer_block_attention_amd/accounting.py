"""Work accounting for reports and sampling: block lists, useful flops, bytes.

Counting only; nothing here takes part in computing the sub-layer.
"""
from __future__ import annotations

import numpy as np


def block_table(lengths, block_frames: int):
    """(start_row, length) of every block, sequence by sequence, in packed order.

    Blocks are non-overlapping runs of `block_frames` frames that restart at each
    sequence's first frame; a sequence's last block holds the remainder.
    """
    out = []
    start = 0
    for ln in np.asarray(lengths, dtype=np.int64):
        ln = int(ln)
        for j in range(0, ln, block_frames):
            out.append((start + j, min(block_frames, ln - j)))
        start += ln
    return out


def sum_block_sq(lengths, block_frames: int) -> int:
    return sum(l * l for _, l in block_table(lengths, block_frames))


def useful_flops(lengths, d_model: int, block_frames: int) -> dict:
    """Useful MFMA flops of one layer: projections 8*N*d^2, attention 4*d*sum L_b^2."""
    n = int(np.sum(lengths))
    sl2 = sum_block_sq(lengths, block_frames)
    qkv = 6 * n * d_model * d_model
    attn = 4 * d_model * sl2
    out = 2 * n * d_model * d_model
    return {"qkv_proj": qkv, "block_attn": attn, "out_proj": out, "total": qkv + attn + out}


def algorithmic_bytes(n_frames: int, d_model: int, elem: int) -> dict:
    """Bytes each kernel must move at minimum (elem = bytes per element).

    qkv_proj reads x and Wqkv and writes Q|K|V; block_attn reads Q|K|V and writes
    O; out_proj reads O, Wo and the residual x and writes out.
    """
    n, d = int(n_frames), int(d_model)
    qkv = elem * (n * d + 3 * d * d + 3 * n * d)
    attn = elem * (3 * n * d + n * d)
    out = elem * (n * d + d * d + n * d + n * d)
    whole = elem * (2 * n * d + 4 * d * d)
    return {"qkv_proj": qkv, "block_attn": attn, "out_proj": out, "layer_min": whole}

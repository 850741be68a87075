"""CPU oracle for the BPE head's posterior-weighted pooling and CTC greedy
decoding.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product package never imports this.

What it computes:
  * pooling (IBM model card, "Model Architecture" (1): the BPE head pools
    with a window of 4 frames, weighting frames by 1 - blank probability of
    a middle layer).  The stride and the normalisation are not on the pages;
    the ONNX export's parity table (its README, "Parity") lists 211 BPE
    positions for the 422-frame clip, i.e. stride 2.  Readings: position j
    of a sequence of T frames pools frames 2j .. min(2j + 4, T) - 1,
    j = 0 .. ceil(T / 2) - 1; the pooled score of class c is
    sum_t w_t * logit[t][c] with w_t = 1 - blank_prob[t], frames in order;
    the positive normaliser 1 / sum_t w_t is left out (it changes no
    argmax).
  * decoding (the Q4 export's README, "Inference note (NAR decode)": the
    head has vocab + 1 = 100353 classes with the blank at 0; per-frame
    argmax, merge consecutive repeats, drop blanks, subtract 1 to get the LLM
    token).  Here "per frame" is per pooled position.  Ties go to the lowest
    class index.

The argmax is an integer decided by floating point, so it is taken in the
kernel's precision: each product w_t * logit and each partial sum is rounded
to IEEE float32 (numpy float32 arithmetic, no fused multiply-add), summed in
frame order, logits widened exactly from bf16.  Pinned in tests/pins.py
(constructed winners with a known decoded sequence, a hand-worked fixture
in tests/golden/, tie and shift rules).
"""
from __future__ import annotations

import numpy as np


def positions(lengths, stride: int = 2):
    """Pooled positions per sequence, ceil(len / stride)."""
    lengths = np.asarray(lengths, np.int64)
    return (lengths + stride - 1) // stride


def pooled_argmax(logits, blank_prob, cu, window: int = 4, stride: int = 2):
    """argmax class of every pooled position, sequence by sequence, int64 [P]."""
    logits = np.asarray(logits, np.float32)
    w = np.float32(1.0) - np.asarray(blank_prob, np.float32)
    cu = np.asarray(cu, np.int64)
    out = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for j in range(int(positions([b - a], stride)[0])):
            t0 = a + stride * j
            t1 = min(t0 + window, b)
            acc = np.zeros(logits.shape[1], np.float32)
            for t in range(t0, t1):
                acc = (acc + w[t] * logits[t]).astype(np.float32)
            out.append(int(np.argmax(acc)))  # first index of the maximum
    return np.asarray(out, np.int64)


def ctc_greedy(ids, pos_lengths, blank: int = 0):
    """Per sequence: merge consecutive repeats, drop blanks, subtract 1.
    Returns (tokens per sequence as a list of int64 arrays)."""
    ids = np.asarray(ids, np.int64)
    out, p = [], 0
    for n in np.asarray(pos_lengths, np.int64):
        seq = ids[p:p + n]
        p += n
        keep = [int(c) - 1 for j, c in enumerate(seq)
                if c != blank and (j == 0 or c != seq[j - 1])]
        out.append(np.asarray(keep, np.int64))
    return out

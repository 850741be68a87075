"""The pooled argmax is decided in fp32 (the oracle and the kernel round each
product and partial sum the same way, so the GPU tests can compare integers
exactly).  This checks that reading against the fp64 pooled scores of the
definition at the class count of the BPE head (100 353 classes, the Q4
export's "Inference note (NAR decode)"): wherever the fp64 winner leads by
more than the fp32 rounding bound, the fp32 argmax is the fp64 argmax; the
remaining positions are near-ties, where either class is a correct answer
to the rounding of the pooled score.  CPU only."""
import numpy as np
import torch

from oracle import ctc_pool as cp
from tests import pins


def test_fp32_argmax_is_the_fp64_argmax_outside_near_ties():
    rng = np.random.default_rng(5)
    classes = 100353
    lengths = [23, 40, 1, 0, 17]  # 41 positions, window 4, stride 2
    n = sum(lengths)
    # the benchmark's distribution: N(0, 1) in bf16, the blank raised by 2
    logits = torch.from_numpy(rng.standard_normal((n, classes)).astype(np.float32))
    logits[:, 0] += 2.0
    logits = logits.to(torch.bfloat16).float().numpy()
    bp = rng.uniform(0, 1, n).astype(np.float32)
    got = cp.pooled_argmax(logits, bp, np.concatenate([[0], np.cumsum(lengths)]))
    s64, bound = pins.pooled_scores_f64(logits, bp, lengths)
    ok, top = pins.decisive(s64, bound)
    near = int((~ok).sum())
    print(f"positions={len(top)} decisive={int(ok.sum())} near-ties={near} "
          f"fp32==fp64 at near-ties: {int((got[~ok] == top[~ok]).sum())}/{near}")
    assert np.array_equal(got[ok], top[ok])
    assert near <= len(top) // 10

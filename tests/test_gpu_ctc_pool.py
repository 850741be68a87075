"""GPU parity of the BPE head's posterior-weighted pooling and CTC greedy
decoding (gs_bpe_pool_ctc_greedy) against its CPU oracle
(oracle/ctc_pool.py), through the C ABI.  Integer outputs: bit-exact."""
import numpy as np
import pytest
import torch

from conformer_block_attention_amd import gsattn, workloads
from oracle import ctc_pool as cp
from tests import gpu_common as G
from tests import pins

pytestmark = pytest.mark.gpu


def _run(logits_f32, bp, lengths, classes, ld, window=4, stride=2):
    """Device run of host arrays: logits [N, classes] (bf16-exact values)."""
    n = logits_f32.shape[0]
    pad = np.zeros((n, ld), np.float32)
    pad[:, :classes] = logits_f32
    dev = G.dev()
    lg = torch.from_numpy(pad).to(torch.bfloat16).to(dev)
    cu = torch.from_numpy(workloads.cu_seqlens(lengths)).to(dev)
    npos = int(cp.positions(lengths, stride).sum())
    am, tok, cnt = gsattn.bpe_pool_ctc_greedy(lg, torch.from_numpy(np.asarray(bp, np.float32)).to(dev),
                                              cu, classes, npos, window=window, stride=stride)
    torch.cuda.synchronize()
    return am.cpu().numpy(), tok.cpu().numpy(), cnt.cpu().numpy()


def _tokens(tok, cnt, lengths, stride=2):
    first = np.concatenate([[0], np.cumsum(cp.positions(lengths, stride))])
    return [tok[first[s]:first[s] + cnt[s]].tolist() for s in range(len(lengths))]


def test_ctc_pool_golden_fixture():
    classes, lengths, bp, logits, argmax, tokens = pins.read_ctc_golden()
    G.print_case("ctc golden", lengths=lengths, classes=classes)
    am, tok, cnt = _run(logits.astype(np.float32), bp, lengths, classes, ld=8)
    assert am.tolist() == argmax
    assert _tokens(tok, cnt, lengths) == tokens


@pytest.mark.parametrize("classes,ld,lengths,window,stride", [
    (1000, 1000, [1, 2, 3, 7, 0, 64, 65], 4, 2),
    (1003, 1008, [40, 9], 4, 2),        # a partial last chunk of classes
    (2048, 2048, [33, 1], 8, 3),        # other window and stride
    (64, 64, [200], 1, 1),              # per-frame argmax
])
def test_ctc_pool_random_exact(classes, ld, lengths, window, stride):
    """Random bf16 logits with a raised blank and random blank probabilities:
    argmax and tokens equal the oracle's exactly."""
    G.print_case("ctc random", classes=classes, ld=ld, lengths=lengths, window=window,
                 stride=stride)
    rng = np.random.default_rng(classes + sum(lengths))
    n = sum(lengths)
    logits = rng.standard_normal((n, classes)).astype(np.float32)
    logits[:, 0] += 1.5
    logits = torch.from_numpy(logits).to(torch.bfloat16).float().numpy()
    bp = rng.uniform(0, 1, n).astype(np.float32)
    am, tok, cnt = _run(logits, bp, lengths, classes, ld, window, stride)
    cu = workloads.cu_seqlens(lengths)
    ref = cp.pooled_argmax(logits, bp, cu, window, stride)
    assert np.array_equal(am, ref)
    want = [t.tolist() for t in cp.ctc_greedy(ref, cp.positions(lengths, stride))]
    assert _tokens(tok, cnt, lengths, stride) == want


def test_ctc_pool_ties_go_to_the_lowest_class():
    """Integer logits with many equal pooled scores (spread over different
    threads' class chunks)."""
    rng = np.random.default_rng(4)
    classes, lengths = 4096, [30, 17]
    n = sum(lengths)
    logits = rng.integers(0, 3, size=(n, classes)).astype(np.float32)
    bp = np.zeros(n, np.float32)
    am, _, _ = _run(logits, bp, lengths, classes, classes)
    ref = cp.pooled_argmax(logits, bp, workloads.cu_seqlens(lengths))
    assert np.array_equal(am, ref)


def test_ctc_pool_full_size():
    """The benchmark's workload (55 093 frames of 100 353 classes, rows of
    100 360): every pooled position's argmax and every sequence's tokens
    against the oracle exactly (each sequence's frames copied back in turn),
    run-to-run equality."""
    lengths = workloads.WORKLOADS["bf16_b128_lognormal"].lengths()
    logits, bp, cu = workloads.bpe_inputs(lengths)
    G.print_case("ctc full", frames=int(cu[-1]), classes=workloads.BPE_CLASSES)
    npos = cp.positions(lengths)
    p = int(npos.sum())
    am, tok, cnt = gsattn.bpe_pool_ctc_greedy(logits, bp, cu, workloads.BPE_CLASSES, p)
    am2, tok2, cnt2 = gsattn.bpe_pool_ctc_greedy(logits, bp, cu, workloads.BPE_CLASSES, p)
    torch.cuda.synchronize()
    assert torch.equal(am, am2) and torch.equal(cnt, cnt2)
    am, tok, cnt = am.cpu().numpy(), tok.cpu().numpy(), cnt.cpu().numpy()
    first = np.concatenate([[0], np.cumsum(npos)])
    # (entries past a sequence's token count are unspecified)
    tok2 = tok2.cpu().numpy()
    for s in range(len(lengths)):
        assert np.array_equal(tok[first[s]:first[s] + cnt[s]], tok2[first[s]:first[s] + cnt[s]])
    cuh = workloads.cu_seqlens(lengths)
    bph = bp.cpu().numpy()
    near = 0
    for s in range(len(lengths)):
        a, b = int(cuh[s]), int(cuh[s + 1])
        lg = logits[a:b, :workloads.BPE_CLASSES].float().cpu().numpy()
        ref = cp.pooled_argmax(lg, bph[a:b], [0, b - a])
        assert np.array_equal(am[first[s]:first[s + 1]], ref), s
        want = cp.ctc_greedy(ref, [len(ref)])[0].tolist()
        assert tok[first[s]:first[s] + cnt[s]].tolist() == want, s
        # the fp32 decision against fp64 pooled scores: equal outside near-ties
        ok, top = pins.decisive(*pins.pooled_scores_f64(lg, bph[a:b], [b - a]))
        assert np.array_equal(am[first[s]:first[s + 1]][ok], top[ok]), s
        near += int((~ok).sum())
    print(f"  sequences={len(lengths)} positions={int(first[-1])} tokens={int(cnt.sum())} "
          f"fp64 near-ties={near}", flush=True)


def test_ctc_pool_num_positions_past_the_count():
    """A num_positions above the sequences' count: the extra positions get
    class 0 and every sequence's tokens are unchanged."""
    rng = np.random.default_rng(8)
    classes, lengths = 256, [9, 4, 0, 13]
    n = sum(lengths)
    logits = torch.from_numpy(rng.standard_normal((n, classes)).astype(np.float32)).to(
        torch.bfloat16)
    bp = torch.from_numpy(rng.uniform(0, 1, n).astype(np.float32))
    dev = G.dev()
    cu = torch.from_numpy(workloads.cu_seqlens(lengths)).to(dev)
    p = int(cp.positions(lengths).sum())
    a1, t1, c1 = gsattn.bpe_pool_ctc_greedy(logits.to(dev), bp.to(dev), cu, classes, p)
    a2, t2, c2 = gsattn.bpe_pool_ctc_greedy(logits.to(dev), bp.to(dev), cu, classes, p + 3)
    torch.cuda.synchronize()
    assert torch.equal(a2[:p], a1) and a2[p:].tolist() == [0, 0, 0]
    assert torch.equal(c2, c1)
    t1, t2, c1 = t1.cpu().numpy(), t2.cpu().numpy(), c1.cpu().numpy()
    first = np.concatenate([[0], np.cumsum(cp.positions(lengths))])
    for s in range(len(lengths)):
        assert np.array_equal(t2[first[s]:first[s] + c1[s]], t1[first[s]:first[s] + c1[s]])

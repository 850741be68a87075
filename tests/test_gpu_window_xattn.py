"""GPU parity of the window cross-attention (gs_window_xattn_fwd) against its
CPU oracle (oracle/window_xattn.py), through the C ABI.  Tolerance: 2e-2 of
the output RMS, as for the bf16 sub-layer (the final rounding of out
dominates)."""
import numpy as np
import pytest
import torch

from conformer_block_attention_amd import gsattn, workloads
from oracle import window_xattn as wx
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _small(lengths, window, nq, f, dq, heads, seed):
    w = workloads.XattnWorkload("small", feat_dim=f, d_q=dq, heads=heads, window_frames=window,
                                queries=nq, seed=seed)
    return workloads.build_xattn_case(w, lengths=lengths)


def _run(c, **kw):
    dev = G.dev()
    out = gsattn.window_xattn_fwd(c.hcat.to(dev), torch.from_numpy(c.cu).to(dev), c.xq.to(dev),
                                  c.wq.to(dev), c.wkv.to(dev), c.wo.to(dev), c.window_frames,
                                  c.heads, **kw)
    torch.cuda.synchronize()
    return out


def _ref(c, windows=None):
    return wx.window_xattn(c.hcat.double().numpy(), c.cu, c.xq.double().numpy(),
                           c.wq.double().numpy(), c.wkv.double().numpy(), c.wo.double().numpy(),
                           c.heads, c.window_frames, windows=windows)


SMALL = [
    # lengths, window, nq, F, dq, heads
    ([31, 15, 4, 0, 16], 15, 3, 256, 256, 2),
    ([1, 2, 3], 1, 3, 128, 256, 2),          # one-frame windows
    ([70, 33], 20, 4, 4096, 256, 2),         # F = 4 x 1024, four queries
    ([300], 15, 1, 64, 512, 4),
    ([47, 200, 9], 64, 2, 192, 256, 2),      # windows longer than a 16-key chunk
]


@pytest.mark.parametrize("lengths,window,nq,f,dq,heads", SMALL)
def test_window_xattn_small(lengths, window, nq, f, dq, heads):
    G.print_case("window_xattn", lengths=lengths, window=window, nq=nq, F=f, dq=dq, heads=heads)
    c = _small(lengths, window, nq, f, dq, heads, seed=sum(lengths) + window)
    got = _run(c).double().cpu().numpy()
    ref = _ref(c)
    err = G.rel_err(got, ref)
    print(f"  windows={c.xq.shape[0]} err={err:.3e}", flush=True)
    assert err <= G.BF16_TOL, err


def test_window_xattn_in_place():
    c = _small([31, 15, 4], 15, 3, 256, 256, 2, seed=9)
    ref = _run(c)
    dev = G.dev()
    xq = c.xq.to(dev)
    out = gsattn.window_xattn_fwd(c.hcat.to(dev), torch.from_numpy(c.cu).to(dev), xq,
                                  c.wq.to(dev), c.wkv.to(dev), c.wo.to(dev), c.window_frames,
                                  c.heads, out=xq)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_window_xattn_full_size():
    """The benchmark's workload and launch configuration (55 093 frames of
    4 096 features, 3 730 windows of 3 queries, dq = 2 048, 16 heads): every
    window against the oracle, run-to-run bit equality, and a sequence run
    alone gives the bits it gets in the batch."""
    name = "bf16_qformer_xattn_b128"
    c = workloads.build_xattn_case(workloads.XATTN_WORKLOADS[name])
    G.print_case(name, frames=int(c.cu[-1]), windows=c.xq.shape[0])
    out = _run(c)
    assert torch.equal(out, _run(c)), "run-to-run results differ"
    nw = c.xq.shape[0]
    ref = _ref(c)
    got = out.double().cpu().numpy()
    err = G.rel_err(got, ref)
    print(f"  windows={nw} err={err:.3e}", flush=True)
    assert err <= G.BF16_TOL, err
    # sequence 5 alone: its windows are a contiguous run of the batch's
    s = 5
    w0 = workloads.num_windows(c.lengths[:s], c.window_frames)
    w1 = w0 + workloads.num_windows(c.lengths[s:s + 1], c.window_frames)
    a, b = int(c.cu[s]), int(c.cu[s + 1])
    dev = G.dev()
    one = gsattn.window_xattn_fwd(c.hcat[a:b].contiguous().to(dev),
                                  torch.tensor([0, b - a], dtype=torch.int32, device=dev),
                                  c.xq[w0:w1].contiguous().to(dev), c.wq.to(dev), c.wkv.to(dev),
                                  c.wo.to(dev), c.window_frames, c.heads)
    torch.cuda.synchronize()
    assert torch.equal(one, out[w0:w1]), "a sequence run alone differs"


def test_window_xattn_debug_check_rejects_a_wrong_window_count(monkeypatch):
    """Under GSATTN_DEBUG_CHECKS=1 a num_windows that is not the sequences'
    count is rejected before any projection runs."""
    monkeypatch.setenv("GSATTN_DEBUG_CHECKS", "1")
    c = _small([31, 15], 15, 3, 256, 256, 2, seed=2)   # 3 + 1 = 4 windows
    dev = G.dev()
    xq = torch.cat([c.xq, c.xq[:1]]).to(dev)            # 5 windows of query states
    with pytest.raises(gsattn.GsError) as e:
        gsattn.window_xattn_fwd(c.hcat.to(dev), torch.from_numpy(c.cu).to(dev), xq,
                                c.wq.to(dev), c.wkv.to(dev), c.wo.to(dev), c.window_frames,
                                c.heads)
    assert "num_windows" in str(e.value)
    out = _run(c)  # the right count passes the check
    assert out.shape == c.xq.shape

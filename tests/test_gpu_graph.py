"""The whole sub-layer captured in a HIP graph (torch.cuda.graph over the
library's launches on the capture stream) and replayed.

The forward enqueues kernels only: no memset, no host synchronisation, no
allocation (the workspace is the caller's, or the static per-GPU array of
the no-allocation entry point).  Each replay runs after eager work on the
same buffers (the output cleared by a fill kernel, the inputs read by other
kernels) and must give the eager result bit for bit, for one layer, for a
two-layer stack whose second layer reuses the first layer's unit table, for
the no-allocation entry point and for the padded-bucket entry point."""
import numpy as np
import pytest
import torch

from conformer_block_attention_amd import gsattn, workloads
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _case(seqs):
    # the first sequences of the headline length mix: ragged blocks, and a
    # projection with a small-tile launch (which builds the unit table)
    lengths = workloads.WORKLOADS[workloads.HEADLINE].lengths()[:seqs]
    return workloads.custom_case(lengths, 1024, 8, 200, torch.bfloat16, seed=11, layers=2)


def _replay_and_check(graph, outs, refs):
    for rep in range(3):
        for o in outs:
            o.fill_(0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {rep} differs from the eager result"


def test_one_layer_and_two_layer_stack_in_a_graph():
    case = _case(40)  # 17 960 frames
    n, d = case.n_frames, case.d_model
    G.print_case("graph_fwd", n=n, S=len(case.lengths))
    x, cu, w1, o1 = G.on_dev(case, 0)
    _, _, w2, o2 = G.on_dev(case, 1)
    ws = gsattn.alloc_workspace(n, d, x.dtype, x.device)
    ref1 = G.run(x, cu, w1, o1, 200, 8, workspace=ws).clone()
    ref2 = G.run(ref1, cu, w2, o2, 200, 8, workspace=ws).clone()

    out1, out2 = torch.empty_like(x), torch.empty_like(x)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gsattn.block_mhsa_fwd(x, cu, w1, o1, 200, 8, out=out1, workspace=ws)
        gsattn.block_mhsa_fwd(out1, cu, w2, o2, 200, 8, out=out2, workspace=ws,
                              reuse_unit_table=True)
    _replay_and_check(g, [out1, out2], [ref1, ref2])


def test_noalloc_entry_point_in_a_graph():
    case = _case(15)  # within the static workspace
    n, d = case.n_frames, case.d_model
    G.print_case("graph_noalloc", n=n, S=len(case.lengths))
    x, cu, w1, o1 = G.on_dev(case, 0)
    ref = G.run(x, cu, w1, o1, 200, 8).clone()
    out = torch.empty_like(x)
    gsattn.block_mhsa_fwd_noalloc(x, cu, w1, o1, 200, 8, out=out)  # the array's address, once
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gsattn.block_mhsa_fwd_noalloc(x, cu, w1, o1, 200, 8, out=out)
    _replay_and_check(g, [out], [ref])


def test_padded_entry_point_in_a_graph():
    """The padded-bucket path (bucket offsets, row table with the unit table,
    the two projections through the row table, the attention and the
    padding-row copy) is kernels only as well: captured and replayed, it
    gives the eager result bit for bit."""
    d, H, B, T = 1024, 8, 200, 512
    lengths = np.array([512, 0, 300, 77, 1, 511, 256, 200], dtype=np.int64)
    S = len(lengths)
    G.print_case("graph_padded", S=S, T=T)
    case = workloads.custom_case(lengths, d, H, B, torch.bfloat16, seed=47)
    wqkv, wo = (w.to(G.dev()) for w in case.weights[0])
    g = torch.Generator(device=G.dev()).manual_seed(47)
    x = torch.randn(S, T, d, generator=g, device=G.dev()).to(torch.bfloat16)
    lens = torch.from_numpy(lengths.astype(np.int32)).to(G.dev())
    ws = torch.empty(gsattn.load().gs_block_mhsa_padded_workspace_bytes(S, T, d, 1),
                     dtype=torch.uint8, device=G.dev())
    ref = gsattn.block_mhsa_fwd_padded(x, lens, wqkv, wo, B, H, workspace=ws).clone()
    out = torch.empty_like(x)
    gsattn.block_mhsa_fwd_padded(x, lens, wqkv, wo, B, H, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gsattn.block_mhsa_fwd_padded(x, lens, wqkv, wo, B, H, out=out, workspace=ws)
    _replay_and_check(graph, [out], [ref])

"""gs_block_mhsa_fwd_noalloc (the library's static per-GPU scratch as the
workspace) against gs_block_mhsa_fwd with a caller workspace, through the C
ABI: bit for bit, on two calls in a row, the second smaller; sizes past the
scratch are refused before any work."""
import pytest
import torch

from conformer_block_attention_amd import gsattn, workloads
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_the_workspace_entry_point(dtype):
    first = workloads.custom_case([3000, 1, 0, 777, 200], 1024, 8, 200, dtype, seed=41)
    second = workloads.custom_case([130, 64, 7], 1024, 8, 200, dtype, seed=42)
    for case in (first, second):  # the second call reuses the scratch, smaller
        G.print_case("noalloc", dtype=dtype, lengths=list(case.lengths))
        x, cu, wqkv, wo = G.on_dev(case)
        got = gsattn.block_mhsa_fwd_noalloc(x, cu, wqkv, wo, case.block_frames, case.heads)
        torch.cuda.synchronize()
        want = G.run(x, cu, wqkv, wo, case.block_frames, case.heads)
        assert torch.equal(got, want)
        y = x.clone()  # in place
        gsattn.block_mhsa_fwd_noalloc(y, cu, wqkv, wo, case.block_frames, case.heads, out=y)
        torch.cuda.synchronize()
        assert torch.equal(y, want)


def test_noalloc_refuses_sizes_past_the_scratch():
    lib = gsattn.load()
    n = 8169  # one frame more than the scratch holds at d = 1024 in bf16
    assert lib.gs_block_mhsa_workspace_bytes(n, 1024, gsattn.GS_BF16) > gsattn.NOALLOC_SCRATCH_BYTES
    assert lib.gs_block_mhsa_workspace_bytes(n - 1, 1024, gsattn.GS_BF16) <= \
        gsattn.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(n, 1024, dtype=torch.bfloat16, device=G.dev())
    cu = torch.tensor([0, n], dtype=torch.int32, device=G.dev())
    w = torch.zeros(3 * 1024, 1024, dtype=torch.bfloat16, device=G.dev())
    with pytest.raises(gsattn.GsError) as e:
        gsattn.block_mhsa_fwd_noalloc(x, cu, w, w[:1024], 200, 8)
    assert e.value.status == gsattn.GS_ERR_UNSUPPORTED

"""The bf16 rounding-point emulation used for the 16-layer chain's tolerance."""
import numpy as np

from conformer_block_attention_amd import workloads
from tests import bf16_emulation, gpu_common as G


def test_emulation_error_is_the_output_rounding_scale(orc):
    """On the 800-frame bucket the emulated bf16 path sits below the 2e-2 bar
    but well above fp64 noise: dominated by the final RNE rounding of out,
    at most half an ulp of |out| < 8 relative to RMS(out) ~ 1, i.e. 2^-6."""
    case = workloads.build_case(workloads.WORKLOADS["bf16_t800"])
    wqkv, wo = case.weights[0]
    mask = np.ones(int(case.cu[-1]), np.uint8)
    ref = orc.block_mhsa(case.x, case.cu, wqkv, wo, case.block_frames, case.heads)
    emu = bf16_emulation.block_mhsa_rows(case.x, case.cu, wqkv, wo, case.block_frames, case.heads,
                                         mask)
    err = G.rel_err(emu, ref)
    assert 5e-3 < err < 2e-2, err


def test_emulation_selects_whole_blocks(orc):
    case = workloads.custom_case([30, 7], 128, 1, 16, workloads.torch.bfloat16, seed=5)
    wqkv, wo = case.weights[0]
    mask = np.zeros(37, np.uint8)
    mask[20] = 1
    emu = bf16_emulation.block_mhsa_rows(case.x, case.cu, wqkv, wo, case.block_frames, case.heads,
                                         mask)
    rows = ~np.isnan(emu).any(axis=1)
    assert rows.tolist() == [False] * 16 + [True] * 14 + [False] * 7

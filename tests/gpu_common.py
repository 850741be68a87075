"""Helpers for the GPU parity tests: move a workload to the device, run the HIP
path through the C ABI, compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

from conformer_block_attention_amd import accounting, gsattn

BF16_TOL = 2e-2   # max-abs error relative to RMS(out), bf16 path vs fp64 oracle
F32_TOL = 1e-4    # same, fp32 path


def tol_for(dtype: torch.dtype) -> float:
    return BF16_TOL if dtype == torch.bfloat16 else F32_TOL


def dev():
    return torch.device("cuda:0")


def on_dev(case, layer=0):
    wqkv, wo = case.weights[layer]
    return (case.x.to(dev()), torch.from_numpy(case.cu).to(dev()), wqkv.to(dev()), wo.to(dev()))


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / sqrt(mean(ref^2)) over the compared elements."""
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-30)


def sample_mask(lengths, block_frames: int, n_random: int = 6, seed: int = 0) -> np.ndarray:
    """Rows of a handful of blocks: first, last, two tails, a few random ones."""
    bt = accounting.block_table(lengths, block_frames)
    n = int(np.sum(lengths))
    rng = np.random.default_rng(seed)
    pick = {0, len(bt) - 1}
    tails = [i for i, (_, l) in enumerate(bt) if l < block_frames]
    for i in tails[:1] + tails[-1:]:
        pick.add(i)
    for i in rng.choice(len(bt), size=min(n_random, len(bt)), replace=False):
        pick.add(int(i))
    mask = np.zeros(n, np.uint8)
    for i in pick:
        s, l = bt[i]
        mask[s:s + l] = 1
    return mask


def print_case(name: str, **kw):
    items = " ".join(f"{k}={v}" for k, v in kw.items())
    print(f"[gpu case] {name} {items}", flush=True)


def run(x, cu, wqkv, wo, block_frames, heads, **kw):
    out = gsattn.block_mhsa_fwd(x, cu, wqkv, wo, block_frames, heads, **kw)
    torch.cuda.synchronize()
    return out

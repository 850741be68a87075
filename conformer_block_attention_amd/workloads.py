"""Seeded synthetic workloads for the block-local MHSA sub-layer.

This module only draws random numbers and lays them out; it holds none of the
sub-layer's arithmetic. Both the HIP path and the CPU oracle are fed from here.

Where the shapes come from (IBM Granite-Speech-4.1-2B-NAR pages):
  * model card, "Model Architecture" (1) CTC Speech Encoder: 16-layer conformer,
    80 log-mel bins with 2-frame stacking, block attention over 4-second blocks.
  * ONNX-export README, "Parity": an 8.43 s clip gives 844 mel frames, i.e. a
    100 Hz mel rate; 2-frame stacking halves it to 50 Hz, so one clip of that
    length is 422 encoder frames and a 4-second block is 200 frames.
  * portable-INT4 README, "What Changed" item 4: a fixed [1, 800, 160] encoder
    bucket, i.e. 800 frames (16 s) of 160 = 80 x 2 stacked features.
  * ONNX-export README, "Multi-clip transcript parity": clips of 39 to 94 s,
    i.e. 1950 to 4700 frames.
  * model card, "Additional results": batched inference at batch size 128;
    portable-INT4 README, "Validation": mean utterance 8.47 s, about 425 frames.

The pages measure on LibriSpeech clips and the Open ASR leaderboard sets; none of
that audio is used. These synthetic inputs stand in for it, with the same frame
counts and batch sizes.

Random-number recipe (one documented generator, shared by both sides):
  numpy PCG64 seeded by SeedSequence(seed, spawn_key=(stream,)), with stream
  0 = sequence lengths, 1 = activations x, 2 + 2*l = Wqkv of layer l,
  3 + 2*l = Wo of layer l.  x ~ N(0, 1); weights ~ N(0, 1/d_model), reading the
  second parameter as a variance (std = d_model**-0.5, exactly 1/32 at 1024).
  Values are drawn in float32; bf16 workloads round them to bfloat16 with
  round-to-nearest-even (torch's float->bfloat16 cast) before either side sees
  them, so both sides read identical numbers.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# Frame rate after 2-frame stacking and the block length it implies.
ENCODER_FRAME_HZ = 50
BLOCK_SECONDS = 4
BLOCK_FRAMES = ENCODER_FRAME_HZ * BLOCK_SECONDS  # 200

STREAM_LENGTHS = 0
STREAM_X = 1


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream,))))


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes, dtype and the recipe for its lengths."""

    name: str
    dtype: str                # "fp32" or "bf16"
    length_kind: str          # "fixed" | "uniform" | "lognormal"
    num_seqs: int
    d_model: int = 1024
    heads: int = 8
    block_frames: int = BLOCK_FRAMES
    layers: int = 1
    seed: int = 0
    fixed_length: int = 0     # for "fixed"
    lo: int = 0               # "uniform": closed range [lo, hi]; "lognormal": clip range
    hi: int = 0
    mean: float = 0.0         # "lognormal": arithmetic mean of the unclipped draw
    sigma: float = 0.0        # "lognormal": log-space standard deviation
    bucket_frames: int = 0    # > 0: padded layout, one bucket of this many rows per sequence

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def lengths(self) -> np.ndarray:
        """Valid frames per sequence (for a padded layout, capped at the bucket)."""
        ln = draw_lengths(self)
        return np.minimum(ln, self.bucket_frames) if self.bucket_frames else ln


def draw_lengths(w: Workload) -> np.ndarray:
    """Sequence lengths in generation (packing) order, int64."""
    if w.length_kind == "fixed":
        return np.full(w.num_seqs, w.fixed_length, dtype=np.int64)
    g = _rng(w.seed, STREAM_LENGTHS)
    if w.length_kind == "uniform":
        # integers uniform on the closed range [lo, hi]
        return g.integers(w.lo, w.hi, size=w.num_seqs, endpoint=True).astype(np.int64)
    if w.length_kind == "lognormal":
        # arithmetic mean `mean` => mu = ln(mean) - sigma^2 / 2; round half-even; clip
        mu = math.log(w.mean) - 0.5 * w.sigma * w.sigma
        raw = g.lognormal(mean=mu, sigma=w.sigma, size=w.num_seqs)
        return np.clip(np.rint(raw), w.lo, w.hi).astype(np.int64)
    raise ValueError(f"unknown length kind {w.length_kind!r}")


# The five workloads, in the order the headline configurations are listed,
# then bf16_b32_long_full: the long-clip batch with one block per sequence
# (block_frames above every length), i.e. full bidirectional attention over
# each packed sequence.  The pages run packed, non-causal attention for the
# bidirectional editor (IBM model card, "Usage", installation note on the
# attention backend; "Model Architecture" (3) Bidirectional LLM Editor); its
# widths are not given, so the encoder's d = 1024, 8 heads are kept, with the
# lengths of the multi-clip range.  bf16_bucket800_b128: the fixed-length
# layout of the portable INT4 export (README "What Changed" item 4: a fixed
# bucket of 800 encoder frames), 128 buckets of 800 rows whose valid lengths
# are the headline batch's lengths capped at 800.
WORKLOADS = {
    "fp32_t422": Workload("fp32_t422", "fp32", "fixed", 1, fixed_length=422),
    "bf16_t800": Workload("bf16_t800", "bf16", "fixed", 1, fixed_length=800),
    "bf16_b32_long": Workload("bf16_b32_long", "bf16", "uniform", 32, lo=1950, hi=4700),
    "bf16_b128_lognormal": Workload("bf16_b128_lognormal", "bf16", "lognormal", 128,
                                    lo=100, hi=1750, mean=425.0, sigma=0.35),
    "bf16_b128_chain16": Workload("bf16_b128_chain16", "bf16", "lognormal", 128,
                                  lo=100, hi=1750, mean=425.0, sigma=0.35, layers=16),
    "bf16_b32_long_full": Workload("bf16_b32_long_full", "bf16", "uniform", 32, lo=1950, hi=4700,
                                   block_frames=4700),
    "bf16_bucket800_b128": Workload("bf16_bucket800_b128", "bf16", "lognormal", 128, lo=100,
                                    hi=1750, mean=425.0, sigma=0.35, bucket_frames=800),
}
WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "bf16_b128_lognormal"


def cu_seqlens(lengths) -> np.ndarray:
    """Exclusive prefix sum of lengths, int32 [S+1] (cu[0] = 0, cu[S] = N)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("total frames exceed int32")
    return cu.astype(np.int32)


def normal(seed: int, stream: int, shape, std: float = 1.0) -> torch.Tensor:
    """float32 N(0, std^2) draw from sub-stream `stream` (CPU tensor)."""
    g = _rng(seed, stream)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return torch.from_numpy(a)


def make_x(n_frames: int, d_model: int, dtype: torch.dtype, seed: int = 0) -> torch.Tensor:
    return normal(seed, STREAM_X, (n_frames, d_model)).to(dtype)


def make_weights(d_model: int, dtype: torch.dtype, seed: int = 0, layer: int = 0):
    """(Wqkv [3d, d], Wo [d, d]) in nn.Linear [out, in] layout."""
    std = 1.0 / math.sqrt(d_model)
    wqkv = normal(seed, 2 + 2 * layer, (3 * d_model, d_model), std).to(dtype)
    wo = normal(seed, 3 + 2 * layer, (d_model, d_model), std).to(dtype)
    return wqkv, wo


@dataclasses.dataclass
class Case:
    """Materialised inputs of one workload (CPU tensors)."""

    name: str
    lengths: np.ndarray      # valid frames per sequence
    cu: np.ndarray           # prefix sums of `lengths` (for a packed layout: x's row offsets)
    x: torch.Tensor          # [rows, d]: packed sequences, or len(lengths) buckets of bucket_frames rows
    weights: list            # [(Wqkv, Wo)] per layer
    block_frames: int
    heads: int
    dtype: torch.dtype
    bucket_frames: int = 0   # > 0: padded layout

    @property
    def n_frames(self) -> int:
        return int(self.cu[-1])

    @property
    def d_model(self) -> int:
        return int(self.x.shape[1])


def build_case(w: Workload, layers: Optional[int] = None) -> Case:
    lengths = w.lengths()
    cu = cu_seqlens(lengths)
    n = len(lengths) * w.bucket_frames if w.bucket_frames else int(cu[-1])
    x = make_x(n, w.d_model, w.torch_dtype, w.seed)
    nl = w.layers if layers is None else layers
    weights = [make_weights(w.d_model, w.torch_dtype, w.seed, l) for l in range(nl)]
    return Case(w.name, lengths, cu, x, weights, w.block_frames, w.heads, w.torch_dtype,
                w.bucket_frames)


def custom_case(lengths, d_model: int, heads: int, block_frames: int, dtype: torch.dtype,
                seed: int = 0, layers: int = 1, name: str = "custom") -> Case:
    """Inputs for arbitrary small shapes (tests): same recipe, given lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = cu_seqlens(lengths)
    n = int(cu[-1])
    x = make_x(n, d_model, dtype, seed)
    weights = [make_weights(d_model, dtype, seed, l) for l in range(layers)]
    return Case(name, lengths, cu, x, weights, block_frames, heads, dtype)


# The window cross-attention of the Q-Former projector (IBM model card, "Model
# Architecture" (2)): 15-frame windows of the concatenated states of four
# encoder layers (F = 4 x 1024) reduced to 3 queries each.  The pages give no
# widths: dq = 2048 with 16 heads of 128 is the width at which two layers of
# self-attention, cross-attention (K|V from F = 4096) and a 4x feed-forward
# come to the stated 160 M parameters (about 75 M per layer).  Frames: the
# headline batch's lengths.  Random streams: 1 hcat, 2 Wq, 3 Wkv, 4 Wo, 5 xq;
# weights N(0, 1/fan_in), hcat and xq N(0, 1).
@dataclasses.dataclass(frozen=True)
class XattnWorkload:
    name: str
    lengths_from: str = "bf16_b128_lognormal"
    feat_dim: int = 4096
    d_q: int = 2048
    heads: int = 16
    window_frames: int = 15
    queries: int = 3
    seed: int = 0


@dataclasses.dataclass
class XattnCase:
    name: str
    lengths: np.ndarray
    cu: np.ndarray
    hcat: torch.Tensor        # [N, F] bf16
    xq: torch.Tensor          # [W, nq, dq] bf16
    wq: torch.Tensor          # [dq, dq]
    wkv: torch.Tensor         # [2 dq, F]
    wo: torch.Tensor          # [dq, dq]
    window_frames: int
    heads: int


def num_windows(lengths, window: int) -> int:
    lengths = np.asarray(lengths, np.int64)
    return int(np.sum((lengths + window - 1) // window))


def build_xattn_case(w: XattnWorkload, lengths=None) -> XattnCase:
    if lengths is None:
        lengths = WORKLOADS[w.lengths_from].lengths()
    lengths = np.asarray(lengths, np.int64)
    cu = cu_seqlens(lengths)
    n = int(cu[-1])
    nw = num_windows(lengths, w.window_frames)
    f, dq, bf = w.feat_dim, w.d_q, torch.bfloat16
    hcat = normal(w.seed, 1, (n, f)).to(bf)
    wq = normal(w.seed, 2, (dq, dq), 1.0 / math.sqrt(dq)).to(bf)
    wkv = normal(w.seed, 3, (2 * dq, f), 1.0 / math.sqrt(f)).to(bf)
    wo = normal(w.seed, 4, (dq, dq), 1.0 / math.sqrt(dq)).to(bf)
    xq = normal(w.seed, 5, (nw, w.queries, dq)).to(bf)
    return XattnCase(w.name, lengths, cu, hcat, xq, wq, wkv, wo, w.window_frames, w.heads)


XATTN_WORKLOADS = {"bf16_qformer_xattn_b128": XattnWorkload("bf16_qformer_xattn_b128")}


# Posterior-weighted pooling + CTC greedy decoding of the BPE head (IBM model
# card, "Model Architecture" (1); Q4 export README, "Inference note"): logits
# over 100 353 classes (blank at 0) for the headline batch's frames, rows
# padded to 100 360 columns (16-byte rows).  The logits are too large to draw
# on the host (11 GB), so they come from torch's seeded device generator
# (Philox), N(0, 1) in bf16 with the blank class raised by 2 (most positions
# decode to blank, as in speech); blank probabilities U(0, 1) in fp32 from
# the same generator.  Both sides read the same device values.
BPE_CLASSES = 100353
BPE_LD = 100360


def bpe_inputs(lengths, classes: int = BPE_CLASSES, ld: int = BPE_LD, seed: int = 0,
               device="cuda"):
    """(logits [N, ld] bf16, blank_prob [N] fp32, cu_seqlens [S+1] int32) on `device`."""
    cu = cu_seqlens(lengths)
    n = int(cu[-1])
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    logits = torch.randn((n, ld), generator=g, device=device, dtype=torch.float32)
    logits[:, 0] += 2.0
    logits = logits.to(torch.bfloat16)
    blank = torch.rand((n,), generator=g, device=device, dtype=torch.float32)
    return logits, blank, torch.from_numpy(cu).to(device)

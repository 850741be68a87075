"""The seeded workloads: sizes, and how the full-sequence one relates to the
long-clip batch.  (Host only: no GPU, no oracle.)"""
import numpy as np

from conformer_block_attention_amd import accounting, workloads


def _frames(name):
    return int(np.sum(workloads.WORKLOADS[name].lengths()))


def test_frame_counts_of_the_seeded_batches():
    # the inputs the benchmark and the full-size tests run on; a change in the
    # generator, the seed or the length recipe shows up here first
    assert _frames("fp32_t422") == 422
    assert _frames("bf16_t800") == 800
    assert _frames("bf16_b128_lognormal") == 55093
    assert _frames("bf16_b32_long") == 107713
    assert _frames("bf16_b128_chain16") == 55093


def test_length_ranges():
    ln = workloads.WORKLOADS["bf16_b128_lognormal"].lengths()
    assert len(ln) == 128 and ln.min() >= 100 and ln.max() <= 1750
    lg = workloads.WORKLOADS["bf16_b32_long"].lengths()
    assert len(lg) == 32 and lg.min() >= 1950 and lg.max() <= 4700


def test_full_sequence_workload_is_the_long_batch_with_one_block_per_sequence():
    full = workloads.WORKLOADS["bf16_b32_long_full"]
    long = workloads.WORKLOADS["bf16_b32_long"]
    assert np.array_equal(full.lengths(), long.lengths())
    assert (full.seed, full.d_model, full.heads, full.dtype) == (long.seed, long.d_model,
                                                                 long.heads, long.dtype)
    lengths = full.lengths()
    assert full.block_frames >= lengths.max()
    table = accounting.block_table(lengths, full.block_frames)
    assert len(table) == len(lengths)
    assert [l for _, l in table] == [int(v) for v in lengths]


def test_bucket_workload_caps_the_headline_lengths():
    w = workloads.WORKLOADS["bf16_bucket800_b128"]
    head = workloads.WORKLOADS["bf16_b128_lognormal"].lengths()
    assert w.bucket_frames == 800
    assert np.array_equal(w.lengths(), np.minimum(head, 800))
    assert (head > 800).any()  # the cap matters for some sequences

"""The attention's work-unit table, read back from the workspace after a call.

It is built either by a kernel of its own (the attention stage called alone,
or a whole sub-layer whose projection has no small-tile launch) or by one more
workgroup of the projection's small-tile launch (a whole sub-layer whose row
count leaves a partial round of 256 x 256 tiles).  Each table is checked
against a host enumeration of the blocks and query groups: the same units,
each once, in order of non-increasing key-chunk count, the count in entry 0,
and every overflow flag word clear.  The sub-layer computed either way gives
the same output bit for bit (each unit is computed whole by one workgroup,
whatever the order)."""
import numpy as np
import pytest
import torch

from conformer_block_attention_amd import gsattn, workloads
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

QG, KC = 224, 32  # query rows per unit and keys per chunk of the bf16 attention


def host_units(lengths, B):
    """(row0, L, q0, qn) of every unit: blocks of B rows restarting at each
    sequence, each block cut into groups of at most QG query rows."""
    out, row = [], 0
    for ln in lengths:
        for a in range(0, int(ln), B):
            L = min(B, int(ln) - a)
            out += [(row + a, L, q0, min(QG, L - q0)) for q0 in range(0, L, QG)]
        row += int(ln)
    return out


def has_small_tile_launch(M, Nc, cus):
    """Whether the projection splits off a round of small tiles (the rule of
    the launcher: whole rounds of 256 x 256 tiles, then one round of BM x 128
    tiles with BM in 64..256 that fits on the CUs)."""
    tpp = Nc // 256
    tiles = -(-M // 256) * tpp
    rounds = tiles // cus
    if rounds < 1 or tiles % cus == 0:
        return False
    rest = M - rounds * cus // tpp * 256
    return rest > 0 and any(-(-rest // bm) * (Nc // 128) <= cus for bm in (64, 128, 192, 256))


def _align(n):
    return (n + 255) // 256 * 256


def check_table(ws, off, n, lengths, B):
    t = ws[off:off + 16 * (n + 1)].cpu().view(torch.int32).reshape(-1, 4).numpy()
    ref = host_units(lengths, B)
    count = int(t[0, 0])
    assert count == len(ref), (count, len(ref))
    got = [tuple(int(v) for v in e) for e in t[1:1 + count]]
    assert sorted(got) == sorted(ref)
    cost = [(L + KC - 1) // KC for _, L, _, _ in got]
    assert all(a >= b for a, b in zip(cost, cost[1:]))
    f0 = off + _align(16 * (n + 1))
    assert int(ws[f0:f0 + 8 * count].count_nonzero()) == 0


def _short_lengths():
    """3 000 sequences of 0..20 frames (some empty): more sequences than the
    builder's threads, so both of its passes loop."""
    g = np.random.default_rng(5)
    ln = g.integers(1, 21, size=3000)
    ln[::97] = 0
    return ln


CASES = {
    # name: (lengths, d, heads, B)
    "headline": (workloads.WORKLOADS[workloads.HEADLINE].lengths(), 1024, 8, 200),
    "many_short": (_short_lengths(), 256, 2, 200),
    "long_B500": (workloads.WORKLOADS["bf16_b32_long"].lengths(), 1024, 8, 500),
}


@pytest.mark.parametrize("name", list(CASES))
def test_unit_table_both_builders(name):
    lengths, d, H, B = CASES[name]
    case = workloads.custom_case(lengths, d, H, B, torch.bfloat16, seed=3)
    n = case.n_frames
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    spare = has_small_tile_launch(n, 3 * d, cus)
    G.print_case(f"unit_table[{name}]", n=n, S=len(lengths), B=B, spare_workgroup=spare)
    x, cu, wqkv, wo = G.on_dev(case)

    # whole sub-layer: the table in the workspace after Q|K|V and O
    ws = torch.full((gsattn.workspace_bytes(n, d, torch.bfloat16),), 0xFF, dtype=torch.uint8,
                    device=G.dev())
    out1 = G.run(x, cu, wqkv, wo, B, H, workspace=ws)
    check_table(ws, _align(n * 3 * d * 2) + _align(n * d * 2), n, lengths, B)

    # the stages one by one: the attention stage's own table kernel
    aws = torch.full((int(gsattn.load().gs_block_attn_workspace_bytes(n)),), 0xFF,
                     dtype=torch.uint8, device=G.dev())
    qkv = gsattn.qkv_proj(x, wqkv)
    o = gsattn.block_attn(qkv, cu, H, B, workspace=aws)
    out2 = gsattn.out_proj_residual(o, wo, x)
    torch.cuda.synchronize()
    check_table(aws, 0, n, lengths, B)
    assert torch.equal(out1, out2)


def test_unit_table_cases_cover_both_builders():
    """The sizes above put the table in a spare workgroup for the headline
    batch and the short sequences, and in its own kernel for the other."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    spare = {k: has_small_tile_launch(int(np.sum(v[0])), 3 * v[1], cus) for k, v in CASES.items()}
    print(f"  spare workgroup: {spare}", flush=True)
    if cus == 256:
        assert spare == {"headline": True, "many_short": True, "long_B500": False}

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

QG, QG_SHORT, KC = 224, 96, 32  # query rows per unit (normal, short batches), keys per chunk


def unit_bound(n, S, B, qg):
    """The launcher's bound on the number of units."""
    return n // B + S + (n // qg if B > qg else 0)


def unit_rows(n, S, B, H, cus):
    """Query rows per unit (the launcher's rule): 96 when units of 96 rows
    still give every (unit, head) item a CU of its own, else 224."""
    return QG_SHORT if unit_bound(n, S, B, QG_SHORT) * H <= cus else QG


def host_units(lengths, B, qg=QG):
    """(row0, L, q0, qn) of every unit: blocks of B rows restarting at each
    sequence, each block cut into groups of at most qg query rows."""
    out, row = [], 0
    for ln in lengths:
        for a in range(0, int(ln), B):
            L = min(B, int(ln) - a)
            out += [(row + a, L, q0, min(qg, L - q0)) for q0 in range(0, L, qg)]
        row += int(ln)
    return out


def has_small_tile_launch(M, Nc, cus):
    """Whether the projection runs a round of small tiles (the rule of the
    launcher: whole rounds of 256 x 256 tiles, then one round of BM x 128
    tiles with BM in 64..256 that fits on the CUs; with fewer large tiles than
    CUs, that round takes every row when it fits)."""
    tpp = Nc // 256
    tiles = -(-M // 256) * tpp
    rounds = tiles // cus

    def fits(rows):
        return any(-(-rows // bm) * (Nc // 128) <= cus for bm in (64, 128, 192, 256))

    if rounds < 1:
        return fits(M)
    if tiles % cus == 0:
        return False
    rest = M - rounds * cus // tpp * 256
    return rest > 0 and fits(rest)


def _align(n):
    return (n + 255) // 256 * 256


def check_table(ws, off, n, lengths, B, qg=QG):
    t = ws[off:off + 16 * (n + 1)].cpu().view(torch.int32).reshape(-1, 4).numpy()
    ref = host_units(lengths, B, qg)
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
    "short_800": (np.array([800]), 1024, 8, 200),
}


@pytest.mark.parametrize("name", list(CASES))
def test_unit_table_both_builders(name):
    lengths, d, H, B = CASES[name]
    case = workloads.custom_case(lengths, d, H, B, torch.bfloat16, seed=3)
    n = case.n_frames
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    spare = has_small_tile_launch(n, 3 * d, cus)
    qg = unit_rows(n, len(lengths), B, H, cus)
    G.print_case(f"unit_table[{name}]", n=n, S=len(lengths), B=B, spare_workgroup=spare, qg=qg)
    x, cu, wqkv, wo = G.on_dev(case)

    # whole sub-layer: the table in the workspace after Q|K|V and O
    ws = torch.full((gsattn.workspace_bytes(n, d, torch.bfloat16),), 0xFF, dtype=torch.uint8,
                    device=G.dev())
    out1 = G.run(x, cu, wqkv, wo, B, H, workspace=ws)
    check_table(ws, _align(n * 3 * d * 2) + _align(n * d * 2), n, lengths, B, qg)

    # the stages one by one: the attention stage's own table kernel
    aws = torch.full((int(gsattn.load().gs_block_attn_workspace_bytes(n)),), 0xFF,
                     dtype=torch.uint8, device=G.dev())
    qkv = gsattn.qkv_proj(x, wqkv)
    o = gsattn.block_attn(qkv, cu, H, B, workspace=aws)
    out2 = gsattn.out_proj_residual(o, wo, x)
    torch.cuda.synchronize()
    check_table(aws, 0, n, lengths, B, qg)
    assert torch.equal(out1, out2)


def test_unit_table_cases_cover_both_builders():
    """The sizes above put the table in a spare workgroup for the headline
    batch and the short sequences, and in its own kernel for the other."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    spare = {k: has_small_tile_launch(int(np.sum(v[0])), 3 * v[1], cus) for k, v in CASES.items()}
    print(f"  spare workgroup: {spare}", flush=True)
    if cus == 256:
        assert spare == {"headline": True, "many_short": True, "long_B500": False,
                         "short_800": True}
        rows = {k: unit_rows(int(np.sum(v[0])), len(v[0]), v[3], v[2], cus)
                for k, v in CASES.items()}
        assert rows == {"headline": QG, "many_short": QG, "long_B500": QG, "short_800": QG_SHORT}


def test_short_batch_units_give_the_packed_bits():
    """An 800-frame sequence alone runs its blocks as 96-row units (every
    item on a CU of its own); packed behind the 128-sequence batch it runs
    them as 224-row units.  Each 32-row group of queries is computed whole
    by one wave either way, so its output rows are the same bits."""
    lengths = np.concatenate([[800], workloads.WORKLOADS[workloads.HEADLINE].lengths()])
    case = workloads.custom_case(lengths, 1024, 8, 200, torch.bfloat16, seed=4)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    qg_alone = unit_rows(800, 1, 200, 8, cus)
    G.print_case("short_batch_units", n=case.n_frames, qg_alone=qg_alone)
    x, cu, wqkv, wo = G.on_dev(case)
    packed = G.run(x, cu, wqkv, wo, 200, 8)
    alone = G.run(x[:800].contiguous(), cu[:2].contiguous(), wqkv, wo, 200, 8)
    if cus == 256:
        assert qg_alone == QG_SHORT
    assert torch.equal(alone, packed[:800])
    # the attention stage alone, too (its own table kernel)
    qkv = gsattn.qkv_proj(x[:800].contiguous(), wqkv)
    o_alone = gsattn.block_attn(qkv, cu[:2].contiguous(), 8, 200)
    qkv_p = gsattn.qkv_proj(x, wqkv)
    o_packed = gsattn.block_attn(qkv_p, cu, 8, 200)
    torch.cuda.synchronize()
    assert torch.equal(o_alone, o_packed[:800])

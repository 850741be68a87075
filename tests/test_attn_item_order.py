"""Host model of how the bf16 attention kernel deals its (unit, head) items
to its persistent workgroups.

Items are dealt in snake order over the cost-sorted unit table: round r gives
workgroup w the item r*G + w (even r) or r*G + G-1-w (odd r).  Odd workgroups
run their own items in the reverse order.  The model repeats the
kernel's cursor arithmetic (the round count R of a workgroup from the last,
partial round) and checks that every item is run exactly once, that a
reversed workgroup runs exactly the items of the forward deal, in reverse,
and that the busiest workgroup's cost stays within one item of the mean on a
cost-sorted list."""
import numpy as np
import pytest


def item_at(r, w, G, items):
    """The kernel's cursor: the item of this workgroup's r-th step (or items
    when it has none)."""
    if w & 1:
        rl = items // G
        sl = G - 1 - w if rl & 1 else w
        R = rl + (1 if rl * G + sl < items else 0)
        r = R - 1 - r
    if r < 0:
        return items
    v = r * G + (G - 1 - w if r & 1 else w)
    return v if v < items else items


def forward_items(w, G, items):
    out, r = [], 0
    while True:
        v = r * G + (G - 1 - w if r & 1 else w)
        if v >= items:
            return out
        out.append(v)
        r += 1


def run_order(w, G, items):
    out, r = [], 0
    while True:
        v = item_at(r, w, G, items)
        if v >= items:
            return out
        out.append(v)
        r += 1


@pytest.mark.parametrize("items", [1, 7, 255, 256, 257, 511, 512, 2704, 3001, 5231])
@pytest.mark.parametrize("cus", [256, 80])
def test_every_item_once_and_reversed_groups(items, cus):
    G = min(items, cus)
    seen = np.zeros(items, np.int32)
    for w in range(G):
        got, fwd = run_order(w, G, items), forward_items(w, G, items)
        assert got == (fwd[::-1] if w & 1 else fwd)
        for v in got:
            seen[v] += 1
    assert np.all(seen == 1)


def test_balance_on_sorted_costs():
    """Costs sorted in decreasing order (chunks per unit of the 128-sequence
    batch's blocks, 8 heads): per-workgroup totals are those of the forward
    deal, and the largest is within one item of the mean."""
    g = np.random.default_rng(0)
    units = np.sort(np.concatenate([np.full(210, 7), g.integers(1, 8, size=128)]))[::-1]
    cost = np.repeat(units, 8)
    items, G = len(cost), 256
    tot = np.array([cost[run_order(w, G, items)].sum() for w in range(G)])
    fwd = np.array([cost[forward_items(w, G, items)].sum() for w in range(G)])
    assert np.array_equal(tot, fwd)
    assert tot.max() - tot.mean() <= cost.max()

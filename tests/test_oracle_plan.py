"""Pins for the split-plan definition (CPU only): brute force over cost positions, exact
coverage, sort order and balance bounds."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import plan as op

CASES = [
    dict(seqlens=[4096] * 64, s_q=1, h=128, causal=False, W=256),
    dict(seqlens=[300, 64, 1, 0, 9000, 130], s_q=1, h=128, causal=False, W=7),
    dict(seqlens=[4096] * 4, s_q=16, h=128, causal=True, W=64),
    dict(seqlens=[20, 5, 70, 3], s_q=16, h=16, causal=True, W=5),
    dict(seqlens=[256, 256], s_q=1, h=16, causal=False, W=256),
    dict(seqlens=[1000, 200, 50, 131072, 2048], s_q=1, h=64, causal=False, W=13),
]


def _brute_worker_of_position(x, total, W):
    """Walk the interval boundaries w C / W (exact fractions) to the one holding x."""
    for w in range(W):
        if Fraction(w * total, W) <= x < Fraction((w + 1) * total, W):
            return w
    raise AssertionError("position outside [0, C)")


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("overhead", [0, 2, 5])
def test_plan_covers_every_page_exactly_once_by_brute_force(case, overhead):
    p = op.split_plan(case["seqlens"], case["s_q"], case["h"], case["causal"], case["W"], overhead)
    W = case["W"]
    assert p.active_workers == min(W, 2 * p.total_cost // (2 + overhead))
    seen = {}
    for w in range(W):
        for (k, lo, hi) in op.worker_segments(p, w):
            for j in range(lo, hi):
                assert (k, j) not in seen
                seen[(k, j)] = w
    for k in range(len(p.pages)):
        pk = int(p.pages[k])
        for j in range(pk):
            # page j starts at C_k + j (overhead + pages) / pages
            x = int(p.cost_begin[k]) + Fraction(j * (overhead + pk), pk)
            w = _brute_worker_of_position(x, p.total_cost, p.active_workers)
            assert seen[(k, j)] == w
            assert op.page_worker(p.cost_begin[k], pk, j, overhead, p.total_cost, p.active_workers) == w
        owners = {seen[(k, j)] for j in range(pk)}
        assert int(p.owner[k]) == min(owners)
        assert int(p.nsplits[k]) == len(owners)
        # every worker inside a split item's range has pages of it
        assert owners == set(range(min(owners), max(owners) + 1))
    assert len(seen) == int(np.sum(p.pages))


@pytest.mark.parametrize("case", CASES)
def test_plan_items_sorted_longest_first_stable(case):
    p = op.split_plan(case["seqlens"], case["s_q"], case["h"], case["causal"], case["W"], 2)
    n_tiles = p.n_tiles
    orig = p.seq * n_tiles + p.tile
    for k in range(len(p.pages) - 1):
        assert p.pages[k] > p.pages[k + 1] or (p.pages[k] == p.pages[k + 1] and orig[k] < orig[k + 1])
    assert sorted(orig.tolist()) == list(range(len(case["seqlens"]) * n_tiles))


@pytest.mark.parametrize("case", CASES)
def test_plan_visible_keys_and_pages(case):
    p = op.split_plan(case["seqlens"], case["s_q"], case["h"], case["causal"], case["W"], 2)
    s, h = case["s_q"], case["h"]
    for k in range(len(p.pages)):
        t = case["seqlens"][p.seq[k]]
        rows = range(128 * p.tile[k], min(128 * (p.tile[k] + 1), s * h))
        if case["causal"]:
            vis = max(min(max(t - s + 1 + r // h, 0), t) for r in rows)
        else:
            vis = t
        assert p.vis[k] == vis
        assert p.pages[k] == max(1, -(-vis // 64))


@pytest.mark.parametrize("case", CASES)
def test_plan_slots_and_balance(case):
    W = case["W"]
    p = op.split_plan(case["seqlens"], case["s_q"], case["h"], case["causal"], W, 2)
    assert p.n_slots <= max(0, 2 * W - 2)
    assert int(np.sum(p.nsplits[p.nsplits > 1])) == p.n_slots
    per_worker = [sum(hi - lo for (_, lo, hi) in op.worker_segments(p, w)) for w in range(W)]
    assert max(per_worker) <= -(-p.total_cost // p.active_workers)
    assert all(n == 0 for n in per_worker[p.active_workers:])
    slots = sorted((int(p.slot_base[k]) + i) for k in p.split_items for i in range(int(p.nsplits[k])))
    assert slots == list(range(p.n_slots))


@pytest.mark.parametrize("overhead", [0, 2, 5])
def test_uniform_batch_splits_evenly_whatever_the_overhead(overhead):
    """Equal items: each page costs the same, so 64 items of 64 pages cut into 16 pages per
    worker, 4 parts per item, for any overhead."""
    p = op.split_plan([4096] * 64, 1, 128, False, 256, overhead)
    assert all(n == 4 for n in p.nsplits)
    assert list(p.owner) == [4 * k for k in range(64)]
    per_worker = [sum(hi - lo for (_, lo, hi) in op.worker_segments(p, w)) for w in range(256)]
    assert set(per_worker) == {16}


def test_tiny_batch_uses_fewer_workers_than_cost_units():
    """Two items of 4 pages, overhead 2: C = 12, W_eff = floor(24 / 4) = 6; pages start at
    0, 1.5, 3, 4.5 and 6, 7.5, 9, 10.5; intervals of length 2."""
    p = op.split_plan([256, 256], 1, 16, False, 256, 2)
    assert p.total_cost == 12 and p.active_workers == 6
    segs = [op.worker_segments(p, w) for w in range(8)]
    assert segs[:6] == [[(0, 0, 2)], [(0, 2, 3)], [(0, 3, 4)], [(1, 0, 2)], [(1, 2, 3)], [(1, 3, 4)]]
    assert segs[6:] == [[], []]
    assert list(p.owner) == [0, 3] and list(p.nsplits) == [3, 3]

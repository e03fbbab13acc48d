"""Pins for the split-plan definition (CPU only): brute force over cost positions, exact
coverage, sort order and balance bounds."""
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


def _brute_worker_of_positions(total, W):
    """Assign every cost position to a worker by walking the interval boundaries."""
    bounds = [(w * total) // W for w in range(W)] + [total]
    owner = np.empty(total, dtype=np.int64)
    for w in range(W):
        owner[bounds[w]:bounds[w + 1]] = w
    return owner


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("overhead", [0, 2, 5])
def test_plan_covers_every_page_exactly_once_by_brute_force(case, overhead):
    p = op.split_plan(case["seqlens"], case["s_q"], case["h"], case["causal"], case["W"], overhead)
    W = case["W"]
    pos_owner = _brute_worker_of_positions(p.total_cost, min(W, p.total_cost))
    seen = {}
    for w in range(W):
        for (k, lo, hi) in op.worker_segments(p, w):
            for j in range(lo, hi):
                assert (k, j) not in seen
                seen[(k, j)] = w
    for k in range(len(p.pages)):
        for j in range(int(p.pages[k])):
            x = int(p.cost_begin[k]) + overhead + j
            assert seen[(k, j)] == pos_owner[x]
            assert op.worker_of(x, p.total_cost, p.active_workers) == pos_owner[x]
        owners = {seen[(k, j)] for j in range(int(p.pages[k]))}
        assert int(p.owner[k]) == min(owners)
        assert int(p.nsplits[k]) == len(owners)
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


def test_uniform_batch_splits_evenly_without_overhead():
    p = op.split_plan([4096] * 64, 1, 128, False, 256, 0)
    assert all(n == 4 for n in p.nsplits)
    per_worker = [sum(hi - lo for (_, lo, hi) in op.worker_segments(p, w)) for w in range(256)]
    assert set(per_worker) == {16}

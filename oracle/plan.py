"""Split-plan definition for jagged decode batches (test infrastructure only).

The FlashMLA-2 newsletter page (section "Architectural Analysis") describes a
radix-sorted block scheduler that balances the partitions of the sequences of one
batch across compute units, so that a 128-token sequence and a 128k-token sequence in
the same batch do not leave stragglers. The pages give no more detail; the plan below
is the plainest reading of that description, written out as a definition so that
the device planner can be checked against it bit for bit:

1. Work items. Each sequence i contributes ceil(s_q * h / 128) row tiles of 128
   (query token, head) rows, row = j * h + head. Tile r of sequence i sees
   ``vis`` keys: all t_i, or, causal, t_i - s_q + 1 + j_last (clamped to [0, t_i])
   where j_last is the last query token with a row in the tile. Its page count is
   max(1, ceil(vis / 64)); an item with nothing visible keeps one (empty) page so that
   some worker writes its zero output.
2. Order. Items sorted by page count, longest first; ties keep item order
   (sequence-major, tile-minor). (A stable sort; the device uses an LSD radix sort.)
3. Cost. Item k costs ``c_k = overhead + pages_k`` units, where ``overhead`` stands for
   loading the item's queries and writing its output. C_k is the exclusive prefix sum
   of costs in sorted order and C the total.
4. Workers. The item's overhead is spread evenly over its pages: page j of item k starts
   at the cost position x = C_k + j * c_k / pages_k (a rational number), so a batch of
   equal items cuts into equal page counts whatever the overhead. W_eff =
   min(W, floor(2 C / (2 + overhead))) workers are used; that keeps each worker's
   interval at least as long as one page of any item of two or more pages, so no
   worker inside a split item's range is left without pages. Worker w < W_eff owns the
   pages whose start lies in [w C / W_eff, (w+1) C / W_eff), i.e. worker
   floor(x W_eff / C); workers w >= W_eff are idle. So each worker gets a contiguous
   run of (item, page) pairs, stored as begin (item, page) inclusive and end (item,
   page) exclusive.
5. Splits. An item whose pages span several workers is split; ``owner`` is the worker of
   its page 0, ``nsplits`` the number of workers it spans, and its partial results go to
   workspace slots slot_base .. slot_base + nsplits - 1 (split index = worker - owner).
   slot_base is the exclusive prefix sum of nsplits over split items in sorted order.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np

ROWS_PER_TILE = 128
PAGE = 64


@dataclasses.dataclass
class Plan:
    num_workers: int
    active_workers: int
    overhead: int
    n_tiles: int
    total_cost: int
    # per item, in sorted order
    seq: np.ndarray
    tile: np.ndarray
    vis: np.ndarray
    pages: np.ndarray
    cost_begin: np.ndarray
    owner: np.ndarray
    nsplits: np.ndarray
    slot_base: np.ndarray
    # per worker
    worker_begin: np.ndarray   # [W, 2] (item, page)
    worker_end: np.ndarray     # [W, 2] (item, page), exclusive
    split_items: np.ndarray    # sorted-order item indices with nsplits > 1
    n_slots: int


def items_of(seqlens, s_q: int, h: int, causal: bool):
    rows = s_q * h
    n_tiles = -(-rows // ROWS_PER_TILE)
    out = []
    for i, t in enumerate(np.asarray(seqlens, dtype=np.int64)):
        t = int(t)
        for r in range(n_tiles):
            j_last = (min(ROWS_PER_TILE * (r + 1), rows) - 1) // h
            vis = t if not causal else min(max(t - s_q + 1 + j_last, 0), t)
            pages = max(1, -(-vis // PAGE))
            out.append((i, r, vis, pages))
    return n_tiles, out


def active_workers(total: int, W: int, overhead: int) -> int:
    """W_eff = min(W, floor(2 C / (2 + overhead)))."""
    return min(int(W), (2 * int(total)) // (2 + int(overhead)))


def page_worker(cost_begin: int, pages: int, j: int, overhead: int, total: int, W: int) -> int:
    """floor(x W / C) for the start x = C_k + j (overhead + pages) / pages of page j, in
    integers: floor((C_k pages + j (overhead + pages)) W / (C pages))."""
    num = (int(cost_begin) * int(pages) + int(j) * (int(overhead) + int(pages))) * int(W)
    return num // (int(total) * int(pages))


def split_plan(seqlens, s_q: int, h: int, causal: bool, num_workers: int, overhead: int) -> Plan:
    W_all = int(num_workers)
    n_tiles, items = items_of(seqlens, s_q, h, causal)
    order = sorted(range(len(items)), key=lambda k: (-items[k][3], k))
    srt = [items[k] for k in order]
    n = len(srt)
    cost_begin = np.zeros(n, dtype=np.int64)
    acc = 0
    for k, it in enumerate(srt):
        cost_begin[k] = acc
        acc += overhead + it[3]
    total = acc
    W = active_workers(total, W_all, overhead)
    owner = np.zeros(n, dtype=np.int64)
    nsplits = np.zeros(n, dtype=np.int64)
    for k, it in enumerate(srt):
        first = page_worker(cost_begin[k], it[3], 0, overhead, total, W)
        last = page_worker(cost_begin[k], it[3], it[3] - 1, overhead, total, W)
        owner[k] = first
        nsplits[k] = last - first + 1
    slot_base = np.full(n, -1, dtype=np.int64)
    slots = 0
    split_items = []
    for k in range(n):
        if nsplits[k] > 1:
            slot_base[k] = slots
            slots += int(nsplits[k])
            split_items.append(k)
    wb = np.zeros((W_all, 2), dtype=np.int64)
    we = np.zeros((W_all, 2), dtype=np.int64)

    def start_of(w):
        """First page (in order) whose start position is >= w C / W_eff."""
        if w >= W:
            return (n, 0)
        k = int(np.searchsorted(cost_begin * W, w * total, side="right")) - 1
        c_k = overhead + srt[k][3]
        # smallest j with C_k + j c_k / pages_k >= w C / W_eff
        num = (w * total - int(cost_begin[k]) * W) * srt[k][3]
        j = -(-num // (W * c_k))
        return (k, j) if j < srt[k][3] else (k + 1, 0)

    for w in range(W_all):
        wb[w] = start_of(w)
        we[w] = start_of(w + 1)
    arr = lambda col: np.array([it[col] for it in srt], dtype=np.int64)
    return Plan(num_workers=W_all, active_workers=W, overhead=overhead, n_tiles=n_tiles, total_cost=total,
                seq=arr(0), tile=arr(1), vis=arr(2), pages=arr(3), cost_begin=cost_begin,
                owner=owner, nsplits=nsplits, slot_base=slot_base, worker_begin=wb, worker_end=we,
                split_items=np.array(split_items, dtype=np.int64), n_slots=slots)


def worker_segments(plan: Plan, w: int) -> List[Tuple[int, int, int]]:
    """(sorted item, first page, end page) runs that worker w processes, in order."""
    kb, pb = (int(x) for x in plan.worker_begin[w])
    ke, pe = (int(x) for x in plan.worker_end[w])
    segs = []
    for k in range(kb, min(ke, len(plan.pages) - 1) + 1):
        lo = pb if k == kb else 0
        hi = pe if k == ke else int(plan.pages[k])
        if hi > lo:
            segs.append((k, lo, hi))
    return segs

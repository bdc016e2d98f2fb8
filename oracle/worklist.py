"""Reference tile schedule for the coalesced launch (integer work).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.

The engine "stably schedules and fuses" whole sequences and shards on a
shared rank (pith.science review of arXiv 2608.01150, "What carries the
argument"). The pages give no algorithm; the reading taken here is a
stable longest-processing-time-first (LPT) list schedule:

1. Cut every item into tiles of ``block_m`` query rows x one head, in the
   order (item, head, query block).
2. Cost of a tile = rows * kv_len + c0 (c0: fixed per-tile overhead).
3. Sort by cost, largest first; the sort is stable, so equal costs keep
   the order of step 1.
4. With n_slots > 0, give each tile in that order to the slot with the
   least load so far (lowest slot index on ties). With n_slots == 0 the
   sorted order itself is the schedule (one workgroup per tile).

The backward splits work the other way, along the key/value axis that a
theta k split cuts (same section): a backward tile is ``block_n`` keys of
one item on one head against all of the item's queries, cost = keys *
q_len + c0, scheduled by the same rule. Its tiles are cut in the order
(item, key block, head), so equal-cost ties run through the heads first.

Python's ``sorted`` is stable and the slot search is a plain scan, so the
result can be checked against the C++ builder bit for bit.
"""

from __future__ import annotations

from typing import Iterable, List, NamedTuple, Tuple


class Tile(NamedTuple):
    q_row0: int
    kv_row0: int
    q_rows: int
    kv_len: int
    head: int
    item: int
    cost: int


def cut_tiles(items: Iterable, block_m: int, c0: int) -> List[Tile]:
    tiles = []
    for idx, it in enumerate(items):
        q_off, q_len, kv_off, kv_len, h0, hc = (it.as_tuple() if hasattr(it, "as_tuple")
                                                else tuple(int(x) for x in it))
        for h in range(h0, h0 + hc):
            for r0 in range(0, q_len, block_m):
                rows = min(block_m, q_len - r0)
                tiles.append(Tile(q_off + r0, kv_off, rows, kv_len, h, idx,
                                  rows * kv_len + c0))
    return tiles


def cut_bwd_tiles(items: Iterable, block_n: int, c0: int) -> List[Tile]:
    tiles = []
    for idx, it in enumerate(items):
        q_off, q_len, kv_off, kv_len, h0, hc = (it.as_tuple() if hasattr(it, "as_tuple")
                                                else tuple(int(x) for x in it))
        if q_len == 0:
            continue
        for k0 in range(0, kv_len, block_n):
            keys = min(block_n, kv_len - k0)
            for h in range(h0, h0 + hc):
                tiles.append(Tile(q_off, kv_off + k0, q_len, keys, h, idx, keys * q_len + c0))
    return tiles


def lpt(tiles: List[Tile], n_slots: int) -> Tuple[List[Tile], List[int], List[int]]:
    """Stable LPT of already-cut tiles: (tiles in schedule order, slot_begin
    offsets [n_slots+1], slot loads); for n_slots == 0 the LPT order."""
    order = sorted(tiles, key=lambda t: -t.cost)
    if n_slots == 0:
        return order, [], []
    loads = [0] * n_slots
    per_slot: List[List[Tile]] = [[] for _ in range(n_slots)]
    for t in order:
        s = min(range(n_slots), key=lambda i: (loads[i], i))
        per_slot[s].append(t)
        loads[s] += t.cost
    flat, begin = [], [0]
    for s in range(n_slots):
        flat += per_slot[s]
        begin.append(len(flat))
    return flat, begin, loads


def lpt_schedule(items: Iterable, block_m: int, n_slots: int, c0: int
                 ) -> Tuple[List[Tile], List[int], List[int]]:
    """Forward schedule: (tiles in schedule order, slot_begin offsets
    [n_slots+1], slot loads). For n_slots == 0: (tiles in LPT order, [], [])."""
    return lpt(cut_tiles(items, block_m, c0), n_slots)


def lpt_schedule_bwd(items: Iterable, block_n: int, n_slots: int, c0: int
                     ) -> Tuple[List[Tile], List[int], List[int]]:
    """Backward schedule over key blocks, same rule."""
    return lpt(cut_bwd_tiles(items, block_n, c0), n_slots)

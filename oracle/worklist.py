"""Reference tile schedule for the coalesced launch (integer work).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.

On one rank the engine places whole sequences and shards together, in a
stable order, and runs them as one fused launch (pith.science review of
arXiv 2608.01150, "What carries the argument"). The pages give no algorithm; the reading taken here is a
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

Key split inside a launch (a theta k split of one item on one rank, same
section): with ``kv_chunk`` > 0 an item with queries and more than
kv_chunk keys is cut into n = ceil(kv_len / kv_chunk) key chunks of
ceil(kv_len / n) keys rounded up to a multiple of 64 (the last chunk
shorter; n then recounted). With ``kv_chunk`` = -1 (automatic) only items
with more than 131,072 keys are cut, as by kv_chunk = 65,536 (the threshold
and chunk size are this build's choice, not the pages'). Chunk p of the k-th split item (in item order)
is numbered n_items + (chunks of earlier split items) + p; its tiles are cut
after all unsplit items' tiles, in (chunk, head, query block) order, and
its partial output goes to workspace rows ws_row0 + p * q_len, ws_row0
being the rows of earlier split items.

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


def _tuple(it):
    return it.as_tuple() if hasattr(it, "as_tuple") else tuple(int(x) for x in it)


# kv_chunk = -1 (automatic): items with more than AUTO_MIN_KEYS keys are
# split as by kv_chunk = AUTO_KEYS, shorter ones stay whole
AUTO_MIN_KEYS = 131072
AUTO_KEYS = 65536


def split_parts(q_len: int, kv_len: int, head_cnt: int, kv_chunk: int) -> Tuple[int, int]:
    """(number of key chunks, keys per chunk) of one item; (1, 0) when the
    item is not split."""
    if kv_chunk == -1:
        kv_chunk = AUTO_KEYS if kv_len > AUTO_MIN_KEYS else 0
    if kv_chunk <= 0 or q_len <= 0 or head_cnt <= 0 or kv_len <= kv_chunk:
        return 1, 0
    n = -(-kv_len // kv_chunk)
    chunk = -(-(-(-kv_len // n)) // 64) * 64
    return -(-kv_len // chunk), chunk


def split_plan(items: Iterable, kv_chunk: int):
    """Output map [(o_shift, to_workspace)] per item and chunk, merge list
    [(q_off, ws_row0, q_len, head_begin, head_cnt, n_parts)] and workspace
    rows of the key split."""
    items = [_tuple(it) for it in items]
    outmap = [(0, 0)] * len(items)
    merges, ws = [], 0
    for q_off, q_len, kv_off, kv_len, h0, hc in items:
        n, _ = split_parts(q_len, kv_len, hc, kv_chunk)
        if n == 1:
            continue
        merges.append((q_off, ws, q_len, h0, hc, n))
        outmap += [(ws + p * q_len - q_off, 1) for p in range(n)]
        ws += n * q_len
    return outmap, merges, ws


def cut_tiles(items: Iterable, block_m: int, c0: int, kv_chunk: int = 0) -> List[Tile]:
    items = [_tuple(it) for it in items]
    tiles = []

    def cut(idx, vitem, k0, keys):
        q_off, q_len, kv_off, kv_len, h0, hc = items[idx]
        for h in range(h0, h0 + hc):
            for r0 in range(0, q_len, block_m):
                rows = min(block_m, q_len - r0)
                tiles.append(Tile(q_off + r0, kv_off + k0, rows, keys, h, vitem,
                                  rows * keys + c0))

    plan = [split_parts(it[1], it[3], it[5], kv_chunk) for it in items]
    for idx, it in enumerate(items):
        if plan[idx][0] == 1:
            cut(idx, idx, 0, it[3])
    vitem = len(items)
    for idx, it in enumerate(items):
        n, chunk = plan[idx]
        if n == 1:
            continue
        for p in range(n):
            cut(idx, vitem, p * chunk, min(chunk, it[3] - p * chunk))
            vitem += 1
    return tiles


def cut_bwd_tiles(items: Iterable, block_n: int, c0: int) -> List[Tile]:
    tiles = []
    for idx, it in enumerate(items):
        q_off, q_len, kv_off, kv_len, h0, hc = _tuple(it)
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


def lpt_schedule(items: Iterable, block_m: int, n_slots: int, c0: int, kv_chunk: int = 0
                 ) -> Tuple[List[Tile], List[int], List[int]]:
    """Forward schedule: (tiles in schedule order, slot_begin offsets
    [n_slots+1], slot loads). For n_slots == 0: (tiles in LPT order, [], [])."""
    return lpt(cut_tiles(items, block_m, c0, kv_chunk), n_slots)


def lpt_schedule_bwd(items: Iterable, block_n: int, n_slots: int, c0: int
                     ) -> Tuple[List[Tile], List[int], List[int]]:
    """Backward schedule over key blocks, same rule."""
    return lpt(cut_bwd_tiles(items, block_n, c0), n_slots)

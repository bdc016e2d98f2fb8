"""Pins of the reference LPT schedule: coverage, stability, lower bounds and
Graham's LPT bound against a brute-force optimum on tiny inputs."""

import itertools

import numpy as np
import pytest

from oracle.worklist import cut_bwd_tiles, cut_tiles, lpt_schedule, lpt_schedule_bwd


def _items(rng, n):
    out = []
    q = kv = 0
    for _ in range(n):
        ql, kl = int(rng.integers(0, 400)), int(rng.integers(0, 500))
        h0 = int(rng.integers(0, 3)); hc = int(rng.integers(1, 3))
        out.append((q, ql, kv, kl, h0, hc))
        q += ql; kv += kl
    return out


def test_cover_every_row_head_once():
    rng = np.random.default_rng(0)
    items = _items(rng, 12)
    tiles, begin, loads = lpt_schedule(items, 128, 7, 64)
    cov = {}
    for t in tiles:
        for r in range(t.q_row0, t.q_row0 + t.q_rows):
            cov[(r, t.head)] = cov.get((r, t.head), 0) + 1
    want = {(it[0] + r, h) for it in items for r in range(it[1]) for h in range(it[4], it[4] + it[5])}
    assert set(cov) == want and set(cov.values()) == {1}
    assert begin[0] == 0 and begin[-1] == len(tiles) and len(begin) == 8
    assert loads == [sum(t.cost for t in tiles[begin[s]:begin[s + 1]]) for s in range(7)]


def test_stable_order_and_determinism():
    items = [(0, 256, 0, 300, 0, 2), (256, 256, 300, 300, 0, 2)]  # all tiles cost-equal
    order, _, _ = lpt_schedule(items, 128, 0, 10)
    assert [(t.item, t.head, t.q_row0) for t in order] == [
        (0, 0, 0), (0, 0, 128), (0, 1, 0), (0, 1, 128), (1, 0, 256), (1, 0, 384), (1, 1, 256), (1, 1, 384)]
    assert lpt_schedule(items, 128, 3, 10) == lpt_schedule(items, 128, 3, 10)
    costs = [t.cost for t in lpt_schedule(_items(np.random.default_rng(1), 9), 64, 0, 5)[0]]
    assert costs == sorted(costs, reverse=True)


def _opt_makespan(costs, m):
    best = float("inf")
    for assign in itertools.product(range(m), repeat=len(costs)):
        loads = [0] * m
        for c, s in zip(costs, assign):
            loads[s] += c
        best = min(best, max(loads))
    return best


def test_graham_bound_against_brute_force():
    rng = np.random.default_rng(2)
    for trial in range(40):
        m = int(rng.integers(2, 4))
        n_items = int(rng.integers(1, 4))
        items = []
        q = 0
        for i in range(n_items):
            ql = int(rng.integers(1, 5)) * 32 - int(rng.integers(0, 31))
            items.append((q, ql, 0, int(rng.integers(1, 90)), 0, 1))
            q += ql
        tiles = cut_tiles(items, 32, 3)
        if len(tiles) > 10:
            continue
        _, _, loads = lpt_schedule(items, 32, m, 3)
        opt = _opt_makespan([t.cost for t in tiles], m)
        mk = max(loads)
        assert mk >= opt and mk >= max(t.cost for t in tiles) and mk * m >= sum(t.cost for t in tiles)
        assert mk <= (4 / 3 - 1 / (3 * m)) * opt + 1e-9


def test_empty_and_zero_kv_items():
    tiles, begin, loads = lpt_schedule([(0, 0, 0, 5, 0, 1), (0, 10, 0, 0, 0, 1)], 128, 2, 7)
    assert len(tiles) == 1 and tiles[0].cost == 7 and tiles[0].kv_len == 0
    assert loads == [7, 0]


def test_backward_tiles_cover_every_key_head_pair_once():
    rng = np.random.default_rng(5)
    items = _items(rng, 10)
    tiles, begin, loads = lpt_schedule_bwd(items, 128, 5, 64)
    cov = {}
    for t in tiles:
        assert t.kv_len <= 128 and t.cost == t.kv_len * t.q_rows + 64
        for r in range(t.kv_row0, t.kv_row0 + t.kv_len):
            cov[(t.item, r, t.head)] = cov.get((t.item, r, t.head), 0) + 1
    want = {(i, it[2] + r, h) for i, it in enumerate(items) if it[1] > 0
            for r in range(it[3]) for h in range(it[4], it[4] + it[5])}
    assert set(cov) == want and set(cov.values()) == {1}
    assert loads == [sum(t.cost for t in tiles[begin[s]:begin[s + 1]]) for s in range(5)]


@pytest.mark.parametrize("cfg,kv_chunk", [(0, 64), (0, 100), (3, 27456), (6, -1)])
def test_key_split_covers_every_key_once(cfg, kv_chunk):
    """With a key split every (query row, head, key) triple of every item is
    still covered by exactly one forward tile, and each item's chunk tiles
    write to its own workspace rows."""
    from oracle.worklist import cut_tiles, split_parts, split_plan
    from coalesced_attention_amd import workloads as W
    wl = W.config(cfg)
    items = [it.as_tuple() for it in wl.items]
    tiles = cut_tiles(items, 256, 0, kv_chunk)
    outmap, merges, ws = split_plan(items, kv_chunk)
    n = len(items)
    # chunk item index -> original item
    vit = {}
    v = n
    for idx, it in enumerate(items):
        p, _ = split_parts(it[1], it[3], it[5], kv_chunk)
        if p > 1:
            for _ in range(p):
                vit[v] = idx
                v += 1
    assert v == len(outmap)
    if cfg in (3, 6):
        # count (row-block, head, key) coverage per item by key ranges only
        for idx, it in enumerate(items):
            q_off, q_len, kv_off, kv_len, h0, hc = it
            mine = [t for t in tiles if (t.item == idx or vit.get(t.item) == idx)]
            for h in range(h0, h0 + hc):
                for r0 in range(0, q_len, 256):
                    ranges = sorted((t.kv_row0, t.kv_row0 + t.kv_len) for t in mine
                                    if t.head == h and t.q_row0 == q_off + r0)
                    pos = kv_off
                    for a, b in ranges:
                        assert a == pos and b > a
                        pos = b
                    assert pos == kv_off + kv_len
    else:
        cover = {}
        for t in tiles:
            idx = t.item if t.item < n else vit[t.item]
            for r in range(t.q_row0, t.q_row0 + t.q_rows):
                for kk in range(t.kv_row0, t.kv_row0 + t.kv_len):
                    key = (idx, r, t.head, kk)
                    cover[key] = cover.get(key, 0) + 1
        assert set(cover.values()) == {1}
        want = sum(it[1] * it[3] * it[5] for it in items)
        assert len(cover) == want
    # workspace rows of different split items and chunks do not overlap
    spans = sorted((m[1] + p * m[2], m[1] + (p + 1) * m[2]) for m in merges for p in range(m[5]))
    for (a, b), (c, d) in zip(spans, spans[1:]):
        assert b <= c
    assert (spans[-1][1] if spans else 0) == ws

"""Seeded synthetic workloads for the coalesced attention path.

This module holds no attention arithmetic. It only

* expands a sequence's parallelism configuration theta = (q, h, k) into the
  work item one rank runs (integer bookkeeping; theta and its legality rule
  are from the pith.science review of arXiv 2608.01150, "What carries the
  argument" and "Assumptions": Sec. IV-A, the head-split degree divides the
  number of heads),
* lays out the five synthetic workloads as packed row ranges and work-item
  tables, and
* draws their iid N(0, 1) inputs from seeded, chunked streams and rounds
  them to bf16 (round to nearest even).

Both the fp64 oracle (tests) and the HIP path (binding, bench) take their
inputs from here, so neither depends on the other.

Packed layout: Q is ``[q_rows, H, d]``, K and V are ``[kv_rows, H, d]``,
row-major, one row per token. A work item names a query row range, a key /
value row range and a head range; every (query row, head) pair it names is
computed against exactly its key range.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

# Draw streams: one numpy PCG64 generator per (seed, tensor, row chunk).
# The chunking keeps the draws identical for any number of threads.
TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO = 0, 1, 2, 3
CHUNK_ROWS = 2048


@dataclasses.dataclass(frozen=True)
class Item:
    """One work item: query rows [q_off, q_off+q_len) attend to key/value
    rows [kv_off, kv_off+kv_len) on heads [head_begin, head_begin+head_cnt)."""

    q_off: int
    q_len: int
    kv_off: int
    kv_len: int
    head_begin: int
    head_cnt: int

    def as_tuple(self) -> Tuple[int, int, int, int, int, int]:
        return (self.q_off, self.q_len, self.kv_off, self.kv_len,
                self.head_begin, self.head_cnt)


@dataclasses.dataclass(frozen=True)
class MergeSpec:
    """KV-split partials to combine: part p occupies query rows
    [row0 + p*part_row_stride, +rows) on heads [head_begin, +head_cnt).
    ``ref_q_off`` is where the same queries sit as one whole item, or -1."""

    n_parts: int
    rows: int
    row0: int
    part_row_stride: int
    head_begin: int
    head_cnt: int
    ref_q_off: int
    ref_kv_off: int
    ref_kv_len: int


@dataclasses.dataclass
class Workload:
    index: int
    name: str
    description: str
    num_heads: int
    head_dim: int
    q_rows: int
    kv_rows: int
    items: List[Item]
    # (dst_row, n_rows, src_row): packed Q rows that repeat other rows
    q_copies: List[Tuple[int, int, int]]
    merges: List[MergeSpec]
    draw_fp32: bool  # inputs specified as fp32 draws (the GPU still gets bf16)
    with_dout: bool

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def flops_fwd(self) -> int:
        """4 * q_len * kv_len * head_cnt * d summed over items (two
        contractions, a multiply and an add each)."""
        return sum(4 * it.q_len * it.kv_len * it.head_cnt * self.head_dim
                   for it in self.items)

    def unique_q_rows(self) -> List[Tuple[int, int]]:
        """Row ranges of packed Q that are drawn (not copies), ascending."""
        copied = sorted((d, d + n) for d, n, _ in self.q_copies)
        out, cur = [], 0
        for a, b in copied:
            if a > cur:
                out.append((cur, a))
            cur = max(cur, b)
        if cur < self.q_rows:
            out.append((cur, self.q_rows))
        return out


def split_bounds(length: int, parts: int, index: int) -> Tuple[int, int]:
    """Floor-balanced split of ``length`` into ``parts`` chunks; the first
    ``length % parts`` chunks are one longer. Returns (start, size)."""
    if parts <= 0 or not 0 <= index < parts:
        raise ValueError("bad split")
    base, rem = divmod(length, parts)
    start = index * base + min(index, rem)
    return start, base + (1 if index < rem else 0)


def theta_item(seq_len: int, num_heads: int, theta: Sequence[int],
               rank: Sequence[int], q_off: int, kv_base: int) -> Item:
    """Work item of one rank of a sequence placed with theta = (q, h, k).

    The rank with coordinates (i_q, i_h, i_k) owns query chunk i_q of the
    sequence (stored packed at ``q_off``), head chunk i_h and key/value
    chunk i_k. ``kv_base`` is the packed row of the sequence's key 0, so the
    item's key range is ``kv_base + start(i_k)``. A whole sequence is
    theta = (1, 1, 1). The head-split degree must divide the head count.
    """
    q, h, k = (int(x) for x in theta)
    iq, ih, ik = (int(x) for x in rank)
    if min(q, h, k) < 1:
        raise ValueError("theta degrees must be >= 1")
    if num_heads % h != 0:
        raise ValueError(f"head split {h} does not divide {num_heads} heads")
    if not (0 <= iq < q and 0 <= ih < h and 0 <= ik < k):
        raise ValueError("rank coordinate out of range")
    _, q_len = split_bounds(seq_len, q, iq)
    kv_start, kv_len = split_bounds(seq_len, k, ik)
    hc = num_heads // h
    return Item(q_off, q_len, kv_base + kv_start, kv_len, ih * hc, hc)


def _whole(q_off, kv_off, L, H):
    return theta_item(L, H, (1, 1, 1), (0, 0, 0), q_off, kv_off)


def _config0() -> Workload:
    H, d = 2, 64
    items = [_whole(0, 0, 64, H), _whole(64, 64, 100, H), _whole(164, 164, 256, H),
             theta_item(256, H, (1, 1, 2), (0, 0, 0), 420, 164),
             theta_item(256, H, (1, 1, 2), (0, 0, 1), 676, 164)]
    return Workload(
        0, "tiny-oracle-check",
        "3 packed sequences of 64, 100 and 256 tokens, 2 heads, d=64, plus the "
        "256-token sequence split k=2 over its keys (two query-row copies)",
        H, d, 932, 420, items, [(420, 256, 164), (676, 256, 164)],
        [MergeSpec(2, 256, 420, 256, 0, H, 164, 164, 256)], True, True)


def _config1() -> Workload:
    H, d = 24, 128
    items = [_whole(1024 * i, 1024 * i, 1024, H) for i in range(32)]
    items += [_whole(32768 + 256 * j, 32768 + 256 * j, 256, H) for j in range(16)]
    return Workload(
        1, "image-only",
        "32 whole 1024-token images (512x512, 8x latent, patch 2) + 16 whole "
        "256-token images, 24 heads, d=128",
        H, d, 36864, 36864, items, [], [], False, False)


def _mixed_items(H: int) -> Tuple[List[Item], int, int]:
    items = [theta_item(32760, H, (4, 1, 1), (0, 0, 0), 0, 0)]
    q, kv = 8190, 32760
    for _ in range(24):
        items.append(_whole(q, kv, 1024, H))
        q += 1024
        kv += 1024
    for _ in range(32):
        items.append(_whole(q, kv, 256, H))
        q += 256
        kv += 256
    return items, q, kv


def _config2() -> Workload:
    H, d = 24, 128
    items, qr, kr = _mixed_items(H)
    return Workload(
        2, "mixed-rank-share",
        "one theta=(4,1,1) shard of a 32760-token video (21x30x52 latents): "
        "8190 queries against all 32760 keys, co-located with 24 whole "
        "1024-token and 32 whole 256-token images; 24 heads, d=128",
        H, d, qr, kr, items, [], [], False, False)


def _config3() -> Workload:
    H, d = 24, 128
    L = 219600
    it0 = theta_item(L, H, (8, 2, 2), (0, 0, 0), 0, 0)
    it1 = theta_item(L, H, (8, 2, 2), (0, 0, 1), 27450, 0)
    items = [it0, it1]
    q, kv = 54900, L
    for _ in range(16):
        items.append(_whole(q, kv, 1024, H))
        q += 1024
        kv += 1024
    return Workload(
        3, "kv-split-shard-merge",
        "theta=(8,2,2) shard of a 219600-token video (61x45x80 latents): a "
        "27450-token query chunk on 12 of 24 heads against both 109800-key "
        "halves (two partials, then merged), co-located with 16 whole "
        "1024-token images; d=128",
        H, d, q, kv, items, [(27450, 27450, 0)],
        [MergeSpec(2, 27450, 0, 27450, 0, 12, -1, 0, L)], False, False)


def _config4() -> Workload:
    w = _config2()
    return Workload(
        4, "train-step-mixed",
        "the mixed rank share, forward then backward (dQ, dK, dV) recomputed "
        "from the saved LSE, dO iid N(0,1) bf16",
        w.num_heads, w.head_dim, w.q_rows, w.kv_rows, w.items, [], [], False, True)


def _config5() -> Workload:
    # One rank's share of the four-720p-videos + 200-images batch on 16 ranks:
    # a 10-s 720p video is 41 x 45 x 80 latents (the 61-frame 15-s latent at
    # 10 s), placed theta = (4, 1, 1), with 13 of the 200 images.
    H, d = 24, 128
    L = 41 * 45 * 80
    items = [theta_item(L, H, (4, 1, 1), (0, 0, 0), 0, 0)]
    q, kv = items[0].q_len, L
    for _ in range(13):
        items.append(_whole(q, kv, 1024, H))
        q += 1024
        kv += 1024
    return Workload(
        5, "four-720p-videos-rank-share",
        "one theta=(4,1,1) shard of a 10-s 720p video (41x45x80 latents, 147600 "
        "tokens): 36900 queries against all 147600 keys, co-located with 13 "
        "whole 1024-token images (a 16-rank share of four such videos and 200 "
        "images); 24 heads, d=128",
        H, d, q, kv, items, [], [], False, False)


def _config6() -> Workload:
    # A 10-s 1080p video: 1920 x 1080 at the same 8x latent and patch 2 gives
    # 120 x 68 per frame, 41 frames; placed theta = (8, 2, 1).
    H, d = 24, 128
    L = 41 * 68 * 120
    items = [theta_item(L, H, (8, 2, 1), (0, 0, 0), 0, 0)]
    q, kv = items[0].q_len, L
    for _ in range(8):
        items.append(_whole(q, kv, 1024, H))
        q += 1024
        kv += 1024
    return Workload(
        6, "1080p-shard",
        "theta=(8,2,1) shard of a 10-s 1080p video (41x68x120 latents, 334560 "
        "tokens): 41820 queries on 12 of 24 heads against all 334560 keys, "
        "co-located with 8 whole 1024-token images; d=128",
        H, d, q, kv, items, [], [], False, False)


_BUILDERS = [_config0, _config1, _config2, _config3, _config4, _config5, _config6]
NUM_CONFIGS = len(_BUILDERS)


def config(index: int) -> Workload:
    return _BUILDERS[index]()


# ---------------------------------------------------------------- drawing

def _pool_size() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_normal(seed: int, tensor: int, rows: int, row_shape: Tuple[int, ...],
                row_start: int = 0) -> np.ndarray:
    """iid N(0,1) float32 of shape (rows, *row_shape). Row r of the stream
    comes from generator default_rng([seed, tensor, r // CHUNK_ROWS]); rows
    [row_start, row_start+rows) of the stream are returned."""
    out = np.empty((rows,) + tuple(row_shape), dtype=np.float32)
    if rows == 0:
        return out
    c0, c1 = row_start // CHUNK_ROWS, (row_start + rows - 1) // CHUNK_ROWS

    def fill(c):
        a, b = c * CHUNK_ROWS, (c + 1) * CHUNK_ROWS
        blk = np.random.default_rng([seed, tensor, c]).standard_normal(
            (CHUNK_ROWS,) + tuple(row_shape), dtype=np.float32)
        lo, hi = max(a, row_start), min(b, row_start + rows)
        out[lo - row_start:hi - row_start] = blk[lo - a:hi - a]

    with ThreadPoolExecutor(_pool_size()) as ex:
        list(ex.map(fill, range(c0, c1 + 1)))
    return out


def round_bf16(x: np.ndarray):
    """fp32 numpy -> torch bfloat16 (CPU), round to nearest even."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


@dataclasses.dataclass
class Inputs:
    q: "object"  # torch bf16 [q_rows, H, d] (CPU)
    k: "object"  # torch bf16 [kv_rows, H, d]
    v: "object"
    dout: Optional["object"] = None  # torch bf16 [q_rows, H, d]
    q32: Optional[np.ndarray] = None  # unrounded fp32 draws (draw_fp32 configs)
    k32: Optional[np.ndarray] = None
    v32: Optional[np.ndarray] = None


def make_inputs(wl: Workload, seed: Optional[int] = None, keep_fp32: bool = False,
                q_scale: float = 1.0) -> Inputs:
    """Seeded inputs of a workload. Draw order and streams: unique Q rows
    (ascending packed order), then K, V and dO, each its own stream; copied
    Q rows repeat their source rows. ``q_scale`` multiplies the fp32 Q
    draws before rounding (a 'peaky' variant for tests)."""
    seed = wl.index if seed is None else seed
    H, d = wl.num_heads, wl.head_dim
    uq = wl.unique_q_rows()
    n_unique = sum(b - a for a, b in uq)
    qd = draw_normal(seed, TENSOR_Q, n_unique, (H, d))
    if q_scale != 1.0:
        qd *= np.float32(q_scale)
    q32 = np.empty((wl.q_rows, H, d), dtype=np.float32)
    pos = 0
    for a, b in uq:
        q32[a:b] = qd[pos:pos + b - a]
        pos += b - a
    del qd
    for dst, n, src in wl.q_copies:
        q32[dst:dst + n] = q32[src:src + n]
    k32 = draw_normal(seed, TENSOR_K, wl.kv_rows, (H, d))
    v32 = draw_normal(seed, TENSOR_V, wl.kv_rows, (H, d))
    inp = Inputs(round_bf16(q32), round_bf16(k32), round_bf16(v32))
    if wl.with_dout:
        inp.dout = round_bf16(draw_normal(seed, TENSOR_DO, wl.q_rows, (H, d)))
    if keep_fp32:
        inp.q32, inp.k32, inp.v32 = q32, k32, v32
    return inp


# ------------------------------------------------------------- sampling

def sample_rows(item: Item, seed: int, block: int = 128,
                full_limit: int = 1024) -> np.ndarray:
    """Query rows (offsets within the item) that a check or a timed oracle
    sample covers: every row of items up to ``full_limit`` queries; for
    longer items the first and last row and two seeded random rows of every
    ``block``-row block."""
    if item.q_len <= full_limit:
        return np.arange(item.q_len, dtype=np.int64)
    rng = np.random.default_rng([seed, item.q_off, item.head_begin])
    rows = []
    for b0 in range(0, item.q_len, block):
        b1 = min(item.q_len, b0 + block)
        rows += [b0, b1 - 1]
        rows += list(rng.integers(b0, b1, size=2))
    return np.unique(np.asarray(rows, dtype=np.int64))


def sample_keys(item: Item, seed: int, block: int = 128,
                full_limit: int = 1024) -> np.ndarray:
    """Key rows (offsets within the item) that a gradient check covers: every
    key of items up to ``full_limit`` keys; for longer items the first and
    last key and two seeded random keys of every ``block``-key block (one
    backward key tile)."""
    if item.kv_len <= full_limit:
        return np.arange(item.kv_len, dtype=np.int64)
    rng = np.random.default_rng([seed, item.kv_off, item.head_begin, 1])
    keys = []
    for b0 in range(0, item.kv_len, block):
        b1 = min(item.kv_len, b0 + block)
        keys += [b0, b1 - 1]
        keys += list(rng.integers(b0, b1, size=2))
    return np.unique(np.asarray(keys, dtype=np.int64))

"""fp64 CPU oracle for coalesced attention: forward, KV-split merge, backward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It
shares no code with the HIP path; the two meet only at the seeded inputs.

What it follows
---------------
* Short sequences run whole, side by side with the shards of split sequences
  (newx.sg page "Zellige: Moldable Sequence Placement for Mixed Image-Video
  DiT Training", Abstract). A shard is one split theta = (q, h, k) of a
  sequence's queries, heads and key/value states (pith.science review of
  arXiv 2608.01150, "What carries the argument").
* The attention itself is dense, exact softmax attention (same review,
  "Assumptions", paper Sec. II, which refers the cost to FlashAttention,
  reference [7], "Fast and memory-efficient exact attention with
  IO-awareness"). Exact attention has a plain definition, so this oracle is
  that definition written out in fp64; the max shift below is an exact
  identity, not an approximation.
* Readings where the pages are silent (each listed in the design notes):
  scale 1/sqrt(d); non-causal; LSE is the natural log of the sum of
  exp(scaled score); an item with no keys gives O = 0 and LSE = -inf; a
  k-split's partials combine by weighting each part with exp(LSE_p - LSE),
  which follows from the definition because the parts' key sets are
  disjoint; the backward recomputes the probabilities from the saved LSE.

Parity pins (tests/test_oracle.py): brute force without max shift on the
tiny workload, torch SDPA / logsumexp in float64, closed forms (zero query,
single key, constant V), invariants (key permutation, key shift, V affine,
independence across packed sequences), merge == whole attention, finite
differences and gradient identities for the backward. The sampled forms
(coalesced_forward_rows, attention_backward_sampled) are pinned at packed
offsets and head ranges that do not start at zero: the forward rows against
the pure-Python brute force, the sampled gradients against the full-matrix
backward (itself pinned by finite differences), each with planted indexing
mistakes that the pin must catch. No function here is parity unpinned.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "attention_rows", "coalesced_forward", "coalesced_forward_rows",
    "merge_partials", "attention_backward_item", "attention_backward_sampled",
    "coalesced_backward", "brute_attention_row",
]


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor -> exact float64 copy
        x = x.detach().float().numpy()
    return np.asarray(x, dtype=np.float64)


def attention_rows(q, k, v, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of queries ``q`` [r, d] against keys ``k`` and
    values ``v`` [n, d] for one head, in fp64.

    z = scale * q k^T;  O = softmax(z) v;  LSE = log(sum_j exp(z_j)).
    Returns O [r, d] and LSE [r]. With n == 0, O = 0 and LSE = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    r, d = q.shape
    if k.shape[0] == 0:
        return np.zeros((r, v.shape[1])), np.full(r, -np.inf)
    z = scale * (q @ k.T)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ v) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def coalesced_forward(Q, K, V, items: Iterable, scale: float,
                      chunk: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Run every work item of a packed batch.

    Q [Tq, H, d], K and V [Tk, H, d]. Each item (q_off, q_len, kv_off,
    kv_len, head_begin, head_cnt) computes its query rows against its own
    key range on its heads. Returns O [Tq, H, d] and LSE [Tq, H]; (row,
    head) pairs that no item covers are NaN.
    """
    Tq, H, d = Q.shape
    O = np.full((Tq, H, d), np.nan)
    LSE = np.full((Tq, H), np.nan)
    for it in items:
        q_off, q_len, kv_off, kv_len, h0, hc = _item_tuple(it)
        for h in range(h0, h0 + hc):
            kh = K[kv_off:kv_off + kv_len, h, :]
            vh = V[kv_off:kv_off + kv_len, h, :]
            for r0 in range(0, q_len, chunk):
                r1 = min(q_len, r0 + chunk)
                o, lse = attention_rows(Q[q_off + r0:q_off + r1, h, :], kh, vh, scale)
                O[q_off + r0:q_off + r1, h, :] = o
                LSE[q_off + r0:q_off + r1, h] = lse
    return O, LSE


def coalesced_forward_rows(Q, K, V, item, head: int, rows: Sequence[int],
                           scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """O [len(rows), d] and LSE [len(rows)] for the given query rows (offsets
    within ``item``) on one head: the sampled form of coalesced_forward."""
    q_off, q_len, kv_off, kv_len, h0, hc = _item_tuple(item)
    rows = np.asarray(rows, dtype=np.int64)
    assert h0 <= head < h0 + hc and (rows.size == 0 or (rows.min() >= 0 and rows.max() < q_len))
    return attention_rows(Q[q_off + rows, head, :], K[kv_off:kv_off + kv_len, head, :],
                          V[kv_off:kv_off + kv_len, head, :], scale)


def merge_partials(o_parts, lse_parts) -> Tuple[np.ndarray, np.ndarray]:
    """Combine partial attention results computed over disjoint key sets.

    o_parts [n, ..., d], lse_parts [n, ...]. With M = max_p LSE_p,
    w_p = exp(LSE_p - M) and W = sum_p w_p: LSE = M + log W and
    O = sum_p (w_p / W) O_p. Parts whose LSE is -inf carry weight 0; if all
    are -inf the result is O = 0, LSE = -inf. (Each part's O_p is its own
    softmax average, so re-weighting by its share of the total exp-sum gives
    the softmax over the union of the key sets.)
    """
    o = _f64(o_parts)
    lse = _f64(lse_parts)
    m = lse.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse - m_safe[None])  # exp(-inf) = 0 for empty parts
    wsum = w.sum(axis=0)
    wsum_safe = np.where(empty, 1.0, wsum)
    out = (w[..., None] * o).sum(axis=0) / wsum_safe[..., None]
    out = np.where(empty[..., None], 0.0, out)
    lse_out = np.where(empty, -np.inf, m_safe + np.log(wsum_safe))
    return out, lse_out


def attention_backward_item(q, k, v, do, scale: float):
    """Gradients of one (item, head) through exact attention, recomputing
    the probabilities from the log-sum-exp.

    With z = scale q k^T, P = exp(z - LSE), O = P v:
      D_r  = sum_c dO_rc O_rc
      dV   = P^T dO
      dP   = dO v^T
      dS   = P * (dP - D)
      dQ   = scale dS k,   dK = scale dS^T q.
    Returns (dq, dk, dv, o, lse).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    if k.shape[0] == 0:
        r, d = q.shape
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros((r, v.shape[1])), np.full(r, -np.inf)
    z = scale * (q @ k.T)
    m = z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    p = np.exp(z - lse[:, None])
    o = p @ v
    D = (do * o).sum(axis=1)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - D[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, o, lse


def attention_backward_sampled(q, k, v, do, scale: float, rows: Sequence[int],
                               cols: Sequence[int], chunk: int = 512):
    """The gradients of attention_backward_item at chosen positions only:
    dQ at query rows ``rows`` and dK, dV at key rows ``cols`` (offsets within
    the item), for items too long to hold the whole [q_len, kv_len]
    probability matrix.

    The definitions are those of attention_backward_item. LSE_r and
    D_r = sum_c dO_rc O_rc need row r's whole softmax, so every query row is
    visited, ``chunk`` rows at a time (rows are independent). A sampled key
    column j needs every query row too: dV_j = sum_r P_rj dO_r and
    dK_j = scale sum_r dS_rj q_r are sums over all rows, accumulated chunk by
    chunk. Returns (dq [len(rows), d], dk [len(cols), d], dv [len(cols), d]).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    n_q, d = q.shape
    dq = np.zeros((rows.size, d))
    dk = np.zeros((cols.size, d))
    dv = np.zeros((cols.size, v.shape[1]))
    if k.shape[0] == 0:
        return dq, dk, dv
    for r0 in range(0, n_q, chunk):
        r1 = min(n_q, r0 + chunk)
        z = scale * (q[r0:r1] @ k.T)                 # [c, n_k]
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        l = e.sum(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(l[:, 0])
        o = (e @ v) / l
        D = (do[r0:r1] * o).sum(axis=1)
        # key columns: P and dS of this chunk's rows at the sampled keys
        p_c = np.exp(z[:, cols] - lse[:, None])
        ds_c = p_c * (do[r0:r1] @ v[cols].T - D[:, None])
        dv += p_c.T @ do[r0:r1]
        dk += scale * (ds_c.T @ q[r0:r1])
        # query rows of this chunk that are sampled: full rows of P and dS
        sel = np.nonzero((rows >= r0) & (rows < r1))[0]
        if sel.size:
            lr = rows[sel] - r0
            p_r = np.exp(z[lr] - lse[lr, None])
            ds_r = p_r * (do[rows[sel]] @ v.T - D[lr, None])
            dq[sel] = scale * (ds_r @ k)
    return dq, dk, dv


def coalesced_backward(Q, K, V, dO, items: Iterable, scale: float):
    """Backward of coalesced_forward for a packed batch. Gradients of items
    that share key/value rows add up. Returns dQ [Tq,H,d], dK, dV [Tk,H,d]."""
    dQ = np.zeros(Q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for it in items:
        q_off, q_len, kv_off, kv_len, h0, hc = _item_tuple(it)
        for h in range(h0, h0 + hc):
            dq, dk, dv, _, _ = attention_backward_item(
                Q[q_off:q_off + q_len, h], K[kv_off:kv_off + kv_len, h],
                V[kv_off:kv_off + kv_len, h], dO[q_off:q_off + q_len, h], scale)
            dQ[q_off:q_off + q_len, h] += dq
            dK[kv_off:kv_off + kv_len, h] += dk
            dV[kv_off:kv_off + kv_len, h] += dv
    return dQ, dK, dV


def brute_attention_row(q: Sequence[float], keys: Sequence[Sequence[float]],
                        values: Sequence[Sequence[float]], scale: float):
    """One query row by the textbook formula in pure Python: weights
    w_j = exp(scale * q.k_j) with no max shift, exact sums by math.fsum.
    Returns (O as a list, LSE)."""
    if not keys:
        return [0.0] * (len(values[0]) if values else len(q)), -math.inf
    w = [math.exp(scale * math.fsum(a * b for a, b in zip(q, kj))) for kj in keys]
    total = math.fsum(w)
    d = len(values[0])
    o = [math.fsum(w[j] * values[j][c] for j in range(len(keys))) / total for c in range(d)]
    return o, math.log(total)


def _item_tuple(it) -> Tuple[int, int, int, int, int, int]:
    if hasattr(it, "as_tuple"):
        return it.as_tuple()
    return tuple(int(x) for x in it)

"""Shared helpers of the GPU parity tests: running the HIP path on a
workload and comparing it with the fp64 oracle under the parity gates."""

from __future__ import annotations

import sys
import time
from dataclasses import dataclass, field

import numpy as np

from coalesced_attention_amd import workloads as W

# Parity gates for bf16 inputs with fp32 accumulation.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
# Per-item relative L2 error of O: long key ranges make O small (about
# sqrt(e / kv_len)), so the absolute gates alone would pass an all-zero O.
REL_L2 = 1e-2


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


@dataclass
class Stats:
    max_abs: float = 0.0
    sum_abs: float = 0.0
    count: int = 0
    lse_max_abs: float = 0.0
    worst_rel_l2: float = 0.0
    rows: int = 0
    per_item: dict = field(default_factory=dict)

    def add(self, key, o_gpu, o_ref, lse_gpu, lse_ref):
        assert np.all(np.isfinite(o_gpu)), f"non-finite O in {key}"
        d = np.abs(o_gpu - o_ref)
        self.max_abs = max(self.max_abs, float(d.max(initial=0.0)))
        self.sum_abs += float(d.sum())
        self.count += d.size
        self.rows += o_gpu.shape[0]
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse_gpu), fin), f"LSE finiteness differs in {key}"
        if fin.any():
            self.lse_max_abs = max(self.lse_max_abs, float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()))
        num, den = self.per_item.get(key, (0.0, 0.0))
        self.per_item[key] = (num + float((d ** 2).sum()), den + float((o_ref ** 2).sum()))

    def finish(self):
        for key, (num, den) in self.per_item.items():
            rel = np.sqrt(num / den) if den > 0 else np.sqrt(num)
            self.worst_rel_l2 = max(self.worst_rel_l2, float(rel))
        return self

    @property
    def mean_abs(self) -> float:
        return self.sum_abs / max(1, self.count)

    def assert_gates(self, what: str):
        self.finish()
        log(f"{what}: rows={self.rows} max_abs={self.max_abs:.3e} mean_abs={self.mean_abs:.3e} "
            f"lse_max_abs={self.lse_max_abs:.3e} worst_rel_l2={self.worst_rel_l2:.3e}")
        assert self.max_abs <= MAX_ABS, (what, self.max_abs)
        assert self.mean_abs <= MEAN_ABS, (what, self.mean_abs)
        assert self.lse_max_abs <= LSE_MAX_ABS, (what, self.lse_max_abs)
        assert self.worst_rel_l2 <= REL_L2, (what, self.worst_rel_l2)


def to_device(inp: W.Inputs, device="cuda"):
    return (inp.q.to(device), inp.k.to(device), inp.v.to(device))


def run_fwd(items, q, k, v, num_heads, head_dim, n_slots=256, poison=True, kv_chunk=0):
    """Build a worklist and run the forward; O and LSE start as NaN so that
    unwritten entries stay visible."""
    import torch
    from coalesced_attention_amd import zl
    wl = zl.build_worklist(items, q.shape[0], k.shape[0], num_heads, head_dim, n_slots=n_slots,
                           device=q.device, kv_chunk=kv_chunk)
    o = torch.full((q.shape[0], num_heads, head_dim), float("nan"), device=q.device)
    lse = torch.full((q.shape[0], num_heads), float("nan"), device=q.device)
    zl.coalesced_attn_fwd(wl, q, k, v, o, lse)
    torch.cuda.synchronize()
    return wl, o, lse


def oracle_compare(stats: Stats, items, Qh, Kh, Vh, O, LSE, scale, full_limit=1024, seed=0,
                   heads=None, block=128):
    """Compare GPU O/LSE (numpy) with the oracle on every row of short items
    and on the sampled rows (first, last, two random per ``block``-row block)
    of long ones. Qh/Kh/Vh are the bf16 inputs as float32 numpy arrays."""
    from oracle.attention import coalesced_forward_rows
    for idx, it in enumerate(items):
        if it.q_len == 0 or it.head_cnt == 0:
            continue
        rows = W.sample_rows(it, seed=seed, block=block, full_limit=full_limit)
        hs = range(it.head_begin, it.head_begin + it.head_cnt) if heads is None else heads(it)
        for h in hs:
            for r0 in range(0, len(rows), 1024):
                rr = rows[r0:r0 + 1024]
                o_ref, l_ref = coalesced_forward_rows(Qh, Kh, Vh, it, h, rr, scale)
                stats.add(idx, O[it.q_off + rr, h], o_ref, LSE[it.q_off + rr, h], l_ref)
    return stats

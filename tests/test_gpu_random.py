"""Seeded random work-item tables on the GPU against the fp64 oracle, in full:
ragged lengths (including empty ones), items sharing key/value rows, head
splits of shared query rows, both head dims, random slot counts and random
in-launch key splits; forward (O, LSE) and backward (dQ, dK, dV) through the
C ABI. Sizes stay small enough for the oracle to finish in seconds."""

import math

import numpy as np
import pytest

from coalesced_attention_amd import workloads as W
from oracle import attention as orc

from gpu_util import LSE_MAX_ABS, MAX_ABS, MEAN_ABS, REL_L2, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _random_problem(rng):
    """Items over packed buffers: mostly disjoint query ranges, some sharing
    key/value rows with earlier items, and head-split pairs on shared query
    rows (disjoint heads, different key ranges)."""
    H = int(rng.choice([1, 2, 3, 4, 6]))
    d = int(rng.choice([64, 128]))
    items, q_off, kv_rows = [], 0, 0
    for _ in range(int(rng.integers(1, 7))):
        q_len = int(rng.choice([0, 1, 31, 255, 256, 257]) if rng.random() < 0.3 else rng.integers(1, 700))
        kv_len = int(rng.choice([0, 1, 63, 64, 65]) if rng.random() < 0.3 else rng.integers(1, 1500))
        if kv_rows and rng.random() < 0.3:           # share keys with earlier items
            kv_off = int(rng.integers(0, kv_rows))
            kv_len = min(kv_len, kv_rows - kv_off)
        else:
            kv_off = kv_rows
            kv_rows += kv_len
        if H > 1 and q_len > 0 and rng.random() < 0.3:  # head split of the same query rows
            h = int(rng.integers(1, H))
            items.append(W.Item(q_off, q_len, kv_off, kv_len, 0, h))
            k2 = int(rng.integers(1, 400))
            items.append(W.Item(q_off, q_len, kv_rows, k2, h, H - h))
            kv_rows += k2
        else:
            h0 = int(rng.integers(0, H))
            items.append(W.Item(q_off, q_len, kv_off, kv_len, h0, int(rng.integers(1, H - h0 + 1))))
        q_off += q_len
    return items, q_off + int(rng.integers(0, 5)), max(1, kv_rows), H, d


# A gradient row (over head_dim) is a sum of terms that share one bf16
# coefficient per query or key, so each of its elements carries an error in
# proportion to the row's terms: for gradients the max-abs bound applies as
# |got - ref| <= MAX_ABS + GRAD_MAX_REL * max|ref row|. O and LSE keep the
# forward's absolute bounds.
GRAD_MAX_REL = 1e-2


def _gates(name, got, ref, rel_tol=0.0, absolute=True):
    d = np.abs(got - ref)
    row = np.abs(ref).max(axis=-1, keepdims=True) if ref.size else ref
    mx = float((d - rel_tol * row).max(initial=0.0))
    mean = float(d.mean()) if d.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / den if den > 0 else float(np.linalg.norm(got - ref))
    assert rel <= REL_L2, (name, mx, mean, rel)
    if absolute:
        assert mx <= MAX_ABS and mean <= MEAN_ABS, (name, mx, mean, rel)
    return mx, rel


@pytest.mark.timeout(600)
@pytest.mark.parametrize("seed", range(64))
def test_random_worklists_forward_and_backward_against_oracle(seed):
    from coalesced_attention_amd import zl
    rng = np.random.default_rng(1000 + seed)
    items, q_rows, kv_rows, H, d = _random_problem(rng)
    n_slots = int(rng.choice([0, 1, 7, 64, 256]))
    kv_chunk = int(rng.choice([0, 0, 64, 200, 512]))
    log(f"seed {seed}: {len(items)} items, q_rows {q_rows}, kv_rows {kv_rows}, H {H}, d {d}, "
        f"n_slots {n_slots}, kv_chunk {kv_chunk}")
    g = torch.Generator().manual_seed(seed)
    mk = lambda n: torch.randn((n, H, d), generator=g).to(torch.bfloat16)
    q, k, v, do = mk(q_rows), mk(kv_rows), mk(kv_rows), mk(q_rows)
    dev = torch.device("cuda:0")
    wl = zl.build_worklist(items, q_rows, kv_rows, H, d, n_slots=n_slots, device=dev, kv_chunk=kv_chunk)
    o = torch.full((q_rows, H, d), float("nan"), device=dev)
    lse = torch.full((q_rows, H), float("nan"), device=dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    zl.coalesced_attn_fwd(wl, qd, kd, vd, o, lse)
    dq, dk, dv = zl.coalesced_attn_bwd(wl, qd, kd, vd, o, lse, do.to(dev))
    torch.cuda.synchronize()
    O, L = o.cpu().numpy(), lse.cpu().numpy()
    Qh, Kh, Vh, Gh = (x.double().numpy() for x in (q, k, v, do))
    s = 1 / math.sqrt(d)
    O_ref, L_ref = orc.coalesced_forward(Qh, Kh, Vh, items, s)
    cov = ~np.isnan(L_ref)
    # rows no item covers stay untouched (NaN); covered ones match the oracle
    assert np.array_equal(np.isnan(L), ~cov)
    if cov.any():
        _gates("O", O[cov], O_ref[cov])
        fin = np.isfinite(L_ref) & cov
        assert np.array_equal(np.isneginf(L[cov]), np.isneginf(L_ref[cov]))
        if fin.any():
            assert float(np.abs(L[fin] - L_ref[fin]).max()) <= LSE_MAX_ABS
    rq, rk, rv = orc.coalesced_backward(Qh, Kh, Vh, Gh, items, s)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        got = got.cpu().numpy()
        assert np.isfinite(got).all(), name
        _gates(name, got, ref, GRAD_MAX_REL)


def _larger_problem(rng):
    """Fewer, longer items: many tiles and key blocks per item, ragged
    tails, key rows shared by a second item, and a head split."""
    H = int(rng.choice([4, 8]))
    d = int(rng.choice([64, 128]))
    items, q_off, kv_rows = [], 0, 0
    for _ in range(int(rng.integers(2, 5))):
        q_len = int(rng.integers(200, 2500))
        kv_len = int(rng.integers(300, 4000))
        if kv_rows and rng.random() < 0.3:
            kv_off = int(rng.integers(0, kv_rows))
            kv_len = min(kv_len, kv_rows - kv_off)
        else:
            kv_off = kv_rows
            kv_rows += kv_len
        if rng.random() < 0.3:
            h = int(rng.integers(1, H))
            items.append(W.Item(q_off, q_len, kv_off, kv_len, 0, h))
            items.append(W.Item(q_off, q_len, kv_off, kv_len, h, H - h))
        else:
            items.append(W.Item(q_off, q_len, kv_off, kv_len, 0, H))
        q_off += q_len
    return items, q_off, kv_rows, H, d


@pytest.mark.timeout(900)
@pytest.mark.parametrize("seed", range(16))
def test_larger_random_worklists_forward_and_backward_against_oracle(seed):
    from coalesced_attention_amd import zl
    rng = np.random.default_rng(5000 + seed)
    items, q_rows, kv_rows, H, d = _larger_problem(rng)
    n_slots = int(rng.choice([0, 256]))
    kv_chunk = int(rng.choice([0, 1024]))
    # Sharper softmax rows on some tables: scores spread over tens of units.
    # O and LSE keep every gate. The gradients (8x larger with Q) keep the
    # relative L2 gate but not the absolute ones: the method's
    # D = rowsum(dO * O) takes the forward's
    # O, whose dominant weight carries its bf16 rounding (~2^-9 of V) when the
    # row's shift is not its maximum, and where dP - D cancels in a sharp row
    # that error dominates the gradient row (up to ~60% of a row whose terms
    # are much larger than the row itself; the tensors stay at ~4e-3 relative
    # L2, and with D taken from the same O the rows match to ~2e-3).
    qscale = float(rng.choice([1.0, 3.0, 8.0]))
    log(f"larger seed {seed}: {len(items)} items, q_rows {q_rows}, kv_rows {kv_rows}, H {H}, d {d}, "
        f"n_slots {n_slots}, kv_chunk {kv_chunk}, q scale {qscale}")
    g = torch.Generator().manual_seed(100 + seed)
    mk = lambda n: torch.randn((n, H, d), generator=g).to(torch.bfloat16)
    q, k, v, do = mk(q_rows), mk(kv_rows), mk(kv_rows), mk(q_rows)
    q = (q.float() * qscale).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    wl = zl.build_worklist(items, q_rows, kv_rows, H, d, n_slots=n_slots, device=dev, kv_chunk=kv_chunk)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = zl.coalesced_attn_fwd(wl, qd, kd, vd)
    dq, dk, dv = zl.coalesced_attn_bwd(wl, qd, kd, vd, o, lse, do.to(dev))
    torch.cuda.synchronize()
    Qh, Kh, Vh, Gh = (x.double().numpy() for x in (q, k, v, do))
    s = 1 / math.sqrt(d)
    O_ref, L_ref = orc.coalesced_forward(Qh, Kh, Vh, items, s)
    _gates("O", o.cpu().numpy(), O_ref)
    assert float(np.abs(lse.cpu().numpy() - L_ref).max()) <= LSE_MAX_ABS
    for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv),
                              orc.coalesced_backward(Qh, Kh, Vh, Gh, items, s)):
        got = got.cpu().numpy()
        assert np.isfinite(got).all(), name
        _gates(name, got, ref, GRAD_MAX_REL, absolute=qscale == 1.0)

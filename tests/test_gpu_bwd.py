"""GPU parity of the recompute-from-LSE backward against the fp64 oracle,
through the C ABI: dQ, dK, dV on the tiny workload (items sharing key/value
rows), ragged shapes, and the training-step workload at full size."""

import math
import os

import numpy as np
import pytest

from coalesced_attention_amd import workloads as W
from oracle import attention as orc

from gpu_util import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Gradient gates: the forward's bounds plus a per-tensor relative L2 error
# (gradients of long items are small). A gradient row (one query's dQ, one
# key's dK or dV, over head_dim) is a sum of terms that share one bf16
# coefficient per query or key (dS or P, rounded to ~2^-9 relative), so
# every element of the row carries an error in proportion to the row's
# terms, also an element that cancels to near zero. The max-abs bound
# therefore applies as |got - ref| <= MAX_ABS + MAX_REL * max|ref row|: keys
# that many queries attend to reach rows of |dK|, |dV| up to 15-20, where
# 2e-2 absolute would be a 1e-3 relative bound.
MAX_ABS = 2e-2
MAX_REL = 1e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from coalesced_attention_amd import zl  # noqa: F401


def _run(items, q, k, v, dout, H, d, n_slots=256, kv_chunk=0):
    from coalesced_attention_amd import zl
    wl = zl.build_worklist(items, q.shape[0], k.shape[0], H, d, n_slots=n_slots, device=q.device,
                           kv_chunk=kv_chunk)
    o, lse = zl.coalesced_attn_fwd(wl, q, k, v)
    dq, dk, dv = zl.coalesced_attn_bwd(wl, q, k, v, o, lse, dout)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


class Gate:
    def __init__(self, what):
        self.what = what
        self.stats = {}

    def add(self, name, got, ref):
        d = np.abs(got - ref)
        s = self.stats.setdefault(name, [0.0, 0.0, 0, 0.0, 0.0])
        row = np.abs(ref).max(axis=-1, keepdims=True)
        s[0] = max(s[0], float((d - MAX_REL * row).max(initial=0.0)))
        s[1] += float(d.sum())
        s[2] += d.size
        s[3] += float((d ** 2).sum())
        s[4] += float((ref ** 2).sum())

    def check(self):
        bad = []
        for name, (mx, sm, n, num, den) in self.stats.items():
            mean = sm / max(1, n)
            rel = math.sqrt(num / den) if den > 0 else math.sqrt(num)
            log(f"{self.what} {name}: max(|d| - {MAX_REL} max|ref row|)={mx:.3e} mean_abs={mean:.3e} "
                f"rel_l2={rel:.3e}")
            if not (mx <= MAX_ABS and mean <= MEAN_ABS and rel <= REL_L2):
                bad.append((name, mx, mean, rel))
        assert not bad, (self.what, bad)


def _oracle_all(items, Q, K, V, dO, scale):
    return orc.coalesced_backward(Q, K, V, dO, items, scale)


@pytest.mark.parametrize("kv_chunk", [0, 64])
def test_backward_tiny_workload_shared_kv(kv_chunk):
    """kv_chunk 64: the forward splits and merges key chunks; the backward
    runs the unsplit schedule on the merged O and LSE."""
    wl = W.config(0)
    inp = W.make_inputs(wl)
    q, k, v, g = (x.cuda() for x in (inp.q, inp.k, inp.v, inp.dout))
    dq, dk, dv = _run(wl.items, q, k, v, g, wl.num_heads, wl.head_dim, kv_chunk=kv_chunk)
    Qh, Kh, Vh, Gh = (x.double().numpy() for x in (inp.q, inp.k, inp.v, inp.dout))
    rq, rk, rv = _oracle_all(wl.items, Qh, Kh, Vh, Gh, wl.softmax_scale)
    gate = Gate("config 0 backward")
    gate.add("dQ", dq, rq)
    gate.add("dK", dk, rk)
    gate.add("dV", dv, rv)
    gate.check()


@pytest.mark.parametrize("d", [64, 128])
def test_backward_ragged_and_head_splits(d):
    H = 4
    rng = np.random.default_rng(d + 1)
    cases = [(1, 1), (63, 129), (64, 128), (65, 127), (200, 300), (130, 5), (7, 400)]
    items, q_off, kv_off = [], 0, 0
    for ql, kl in cases:
        items.append(W.Item(q_off, ql, kv_off, kl, 0, H))
        q_off += ql
        kv_off += kl
    items.append(W.Item(q_off, 90, 0, 300, 0, 2))      # shares keys with earlier items
    items.append(W.Item(q_off, 90, 300, 150, 2, 2))    # head split of the same rows
    q_off += 90
    items.append(W.Item(q_off, 40, 0, 0, 0, H))        # no keys: O = 0, no gradient
    items.append(W.Item(q_off + 40, 0, 0, 50, 0, H))   # no queries
    q_off += 40
    mk = lambda n: torch.from_numpy(rng.standard_normal((n, H, d)).astype(np.float32)).to(torch.bfloat16)
    q, k, v, g = mk(q_off), mk(kv_off), mk(kv_off), mk(q_off)
    dq, dk, dv = _run(items, q.cuda(), k.cuda(), v.cuda(), g.cuda(), H, d, n_slots=7)
    rq, rk, rv = _oracle_all(items, q.double().numpy(), k.double().numpy(), v.double().numpy(),
                             g.double().numpy(), 1 / math.sqrt(d))
    gate = Gate(f"ragged d={d} backward")
    gate.add("dQ", dq, rq)
    gate.add("dK", dk, rk)
    gate.add("dV", dv, rv)
    gate.check()


@pytest.mark.parametrize("d", [64, 128])
def test_backward_key_tile_and_step_edges(d):
    """Key counts around the dK/dV tile (256 keys, 32 per wave) and query
    counts giving one to six 32-row steps of either parity, with every item
    reading the same key/value rows so that the dK/dV atomics of all items
    add up in the same rows."""
    H = 2
    rng = np.random.default_rng(40 + d)
    kls = [255, 256, 257, 511, 512, 513]
    qls = [31, 32, 33, 96, 160, 161]
    items, q_off = [], 0
    for ql, kl in zip(qls, kls):
        items.append(W.Item(q_off, ql, 0, kl, 0, H))
        q_off += ql
    kv_rows = max(kls)
    mk = lambda n: torch.from_numpy(rng.standard_normal((n, H, d)).astype(np.float32)).to(torch.bfloat16)
    q, k, v, g = mk(q_off), mk(kv_rows), mk(kv_rows), mk(q_off)
    dq, dk, dv = _run(items, q.cuda(), k.cuda(), v.cuda(), g.cuda(), H, d, n_slots=5)
    rq, rk, rv = _oracle_all(items, q.double().numpy(), k.double().numpy(), v.double().numpy(),
                             g.double().numpy(), 1 / math.sqrt(d))
    gate = Gate(f"tile edges d={d} backward")
    gate.add("dQ", dq, rq)
    gate.add("dK", dk, rk)
    gate.add("dV", dv, rv)
    gate.check()


@pytest.mark.timeout(900)
def test_backward_training_step_full_size():
    """Config 4 at full size: every image item in full on every head; the
    video shard (8190 queries x 32760 keys) on EVERY head at sampled
    positions that touch every tile: dQ at the first, last and two random
    rows of every 128-row block, dK and dV at the first, last and two random
    keys of every 128-key block. The sampled oracle computes LSE and D over
    all of the shard's rows, so each sampled value is exact."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    wl = W.config(4)
    log("drawing inputs of config 4")
    inp = W.make_inputs(wl)
    q, k, v, g = (x.cuda() for x in (inp.q, inp.k, inp.v, inp.dout))
    log("config 4: forward + backward on GPU")
    dq, dk, dv = _run(wl.items, q, k, v, g, wl.num_heads, wl.head_dim)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    Qh, Kh, Vh, Gh = (x.float().numpy() for x in (inp.q, inp.k, inp.v, inp.dout))
    s = wl.softmax_scale
    gate = Gate("config 4 backward")
    # every image item in full, every head
    for it in wl.items[1:]:
        for h in range(it.head_begin, it.head_begin + it.head_cnt):
            qs, ks = slice(it.q_off, it.q_off + it.q_len), slice(it.kv_off, it.kv_off + it.kv_len)
            rq, rk, rv, _, _ = orc.attention_backward_item(Qh[qs, h], Kh[ks, h], Vh[ks, h], Gh[qs, h], s)
            gate.add("dQ", dq[qs, h], rq)
            gate.add("dK", dk[ks, h], rk)
            gate.add("dV", dv[ks, h], rv)
    it = wl.items[0]
    qs, ks = slice(it.q_off, it.q_off + it.q_len), slice(it.kv_off, it.kv_off + it.kv_len)
    heads = list(range(it.head_begin, it.head_begin + it.head_cnt))
    log(f"config 4: images checked; video shard on all {len(heads)} heads (sampled rows and keys)")

    def shard_head(h):
        rows = W.sample_rows(it, seed=100 + h)
        cols = W.sample_keys(it, seed=100 + h)
        ref = orc.attention_backward_sampled(Qh[qs, h], Kh[ks, h], Vh[ks, h], Gh[qs, h], s, rows, cols)
        return h, rows, cols, ref

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        for h, rows, cols, (rq, rk, rv) in ex.map(shard_head, heads):
            gate.add("dQ shard", dq[it.q_off + rows, h], rq)
            gate.add("dK shard", dk[it.kv_off + cols, h], rk)
            gate.add("dV shard", dv[it.kv_off + cols, h], rv)
            # the identities the oracle is pinned by hold on the GPU result too
            assert np.abs(dk[ks, h].sum(0)).max() < 1e-2, h
            np.testing.assert_allclose(dv[ks, h].sum(0), Gh[qs, h].sum(0), atol=2e-2, rtol=1e-3)
    log(f"config 4: shard heads done ({workers} threads)")
    gate.check()


def test_backward_accumulates_into_caller_buffers():
    """dQ, dK, dV are sums into the caller's buffers: a second call adds the
    same gradient again."""
    from coalesced_attention_amd import zl
    wl = W.config(0)
    inp = W.make_inputs(wl)
    q, k, v, g = (x.cuda() for x in (inp.q, inp.k, inp.v, inp.dout))
    built = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim, device=q.device)
    o, lse = zl.coalesced_attn_fwd(built, q, k, v)
    once = [t.clone() for t in zl.coalesced_attn_bwd(built, q, k, v, o, lse, g)]
    bufs = zl.coalesced_attn_bwd(built, q, k, v, o, lse, g)
    twice = zl.coalesced_attn_bwd(built, q, k, v, o, lse, g, *bufs)
    torch.cuda.synchronize()
    for a, b in zip(once, twice):
        torch.testing.assert_close(b, 2 * a, rtol=1e-5, atol=1e-6)


def test_backward_deterministic_over_slot_counts():
    """dQ has one writer per (row, head), and in a workload whose items use
    disjoint key/value rows so do dK and dV: every schedule gives the same
    bits."""
    from coalesced_attention_amd import zl
    items = [W.Item(0, 300, 0, 500, 0, 4), W.Item(300, 128, 500, 128, 0, 4), W.Item(428, 70, 628, 33, 0, 4)]
    rng = np.random.default_rng(11)
    mk = lambda n: torch.from_numpy(rng.standard_normal((n, 4, 128)).astype(np.float32)).to(torch.bfloat16).cuda()
    q, k, v, g = mk(498), mk(661), mk(661), mk(498)
    ref = None
    for n_slots in (256, 97, 0, 1):
        wl = zl.build_worklist(items, 498, 661, 4, 128, n_slots=n_slots, device=q.device)
        o, lse = zl.coalesced_attn_fwd(wl, q, k, v)
        got = [t.cpu() for t in zl.coalesced_attn_bwd(wl, q, k, v, o, lse, g)]
        if ref is None:
            ref = got
        for a, b in zip(ref, got):
            assert torch.equal(a, b), n_slots


@pytest.mark.timeout(600)
def test_backward_long_key_range_offsets_past_2gb():
    """Backward of one 200-query item against 2^20 keys on 4 heads (key
    offsets in bytes pass 2^31), checked on two heads against the oracle."""
    H, d = 4, 128
    n_keys = 1 << 20
    items = [W.Item(0, 200, 0, n_keys, 0, H)]
    g = torch.Generator(device="cuda").manual_seed(6)
    q = torch.randn((200, H, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((n_keys, H, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((n_keys, H, d), generator=g, device="cuda").to(torch.bfloat16)
    do = torch.randn((200, H, d), generator=g, device="cuda").to(torch.bfloat16)
    dq, dk, dv = _run(items, q, k, v, do, H, d)
    Qh, Kh, Vh, Gh = (x.float().cpu().numpy() for x in (q, k, v, do))
    gate = Gate("2^20-key backward")
    for h in (0, 3):
        rq, rk, rv, _, _ = orc.attention_backward_item(Qh[:, h], Kh[:, h], Vh[:, h], Gh[:, h], 1 / math.sqrt(d))
        gate.add("dQ", dq[:, h], rq)
        gate.add("dK", dk[:, h], rk)
        gate.add("dV", dv[:, h], rv)
    gate.check()

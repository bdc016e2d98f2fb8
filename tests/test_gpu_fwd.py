"""GPU parity of the coalesced forward and the partial merge against the fp64
oracle, through the C ABI, plus GPU-side invariants and edge cases."""

import math

import numpy as np
import pytest

from coalesced_attention_amd import workloads as W
from oracle import attention as orc

from gpu_util import LSE_MAX_ABS, Stats, log, oracle_compare, run_fwd, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from coalesced_attention_amd import zl  # noqa: F401  (fails loudly if libzl.so is missing)


_CACHE = {}


def _workload(c):
    if c not in _CACHE:
        _CACHE.clear()
        wl = W.config(c)
        log(f"drawing inputs of config {c} ({wl.name})")
        inp = W.make_inputs(wl)
        _CACHE[c] = (wl, inp, to_device(inp))
    return _CACHE[c]


def _host(x):
    return x.float().numpy()


# ----------------------------------------------------------------- configs

@pytest.mark.timeout(900)
@pytest.mark.parametrize("c,kv_chunk", [(0, 0), (1, 0), (2, 0), (3, 0), (0, 64), (3, 27456), (5, 0),
                                        (6, 0), (6, 65536), (5, -1)])
def test_forward_parity(c, kv_chunk):
    """Every config against the oracle; with kv_chunk > 0 the long items are
    split into key chunks inside the launch and merged (config 3's 109,800
    keys into 4 chunks of 27,456; the 1080p shard's 334,560 keys into 6
    chunks of at most 65,536; the four-720p share's 147,600 keys into 3
    chunks by the automatic split, kv_chunk = -1; config 0's items into
    64-key chunks)."""
    wl, inp, (q, k, v) = _workload(c)
    log(f"config {c}: forward on GPU, {len(wl.items)} items, kv_chunk {kv_chunk}")
    built, o, lse = run_fwd(wl.items, q, k, v, wl.num_heads, wl.head_dim, kv_chunk=kv_chunk)
    if kv_chunk:
        assert built.header.n_merges > 0
    O, LSE = o.cpu().numpy(), lse.cpu().numpy()
    log(f"config {c}: {built.n_tiles} tiles done; oracle check")
    # the second workload's shards (147,600 and 334,560 keys) are checked on
    # 4 rows of every 256-row tile
    st = oracle_compare(Stats(), wl.items, _host(inp.q), _host(inp.k), _host(inp.v), O, LSE,
                        wl.softmax_scale, seed=c, block=256 if c >= 5 else 128)
    st.assert_gates(f"config {c} forward (kv_chunk {kv_chunk})")
    # every covered (row, head) written, nothing else
    cov = np.zeros((wl.q_rows, wl.num_heads), bool)
    for it in wl.items:
        cov[it.q_off:it.q_off + it.q_len, it.head_begin:it.head_begin + it.head_cnt] = True
    assert np.array_equal(~np.isnan(LSE), cov)
    assert np.array_equal(~np.isnan(O).any(-1), cov)
    assert np.array_equal(np.isnan(O).all(-1), ~cov)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("c", [0, 3])
def test_merge_parity(c):
    from coalesced_attention_amd import zl
    wl, inp, (q, k, v) = _workload(c)
    built, o, lse = run_fwd(wl.items, q, k, v, wl.num_heads, wl.head_dim)
    m = wl.merges[0]
    mo, ml = zl.merge_partials(o, lse, m.row0, m.n_parts, m.rows, m.part_row_stride,
                               m.head_begin, m.head_cnt)
    torch.cuda.synchronize()
    MO, ML = mo.cpu().numpy(), ml.cpu().numpy()
    # the merged queries are the partials' shared query rows, against all keys
    whole = W.Item(m.row0, m.rows, m.ref_kv_off, m.ref_kv_len, m.head_begin, m.head_cnt)
    st = Stats()
    rows = W.sample_rows(whole, seed=7, full_limit=1024)
    if c == 3:
        rows = rows[::4]  # full-range oracle rows cost 220k keys each
    Qh, Kh, Vh = _host(inp.q), _host(inp.k), _host(inp.v)
    for h in range(m.head_begin, m.head_begin + m.head_cnt):
        o_ref, l_ref = orc.coalesced_forward_rows(Qh, Kh, Vh, whole, h, rows, wl.softmax_scale)
        st.add(h, MO[rows, h], o_ref, ML[rows, h], l_ref)
    st.assert_gates(f"config {c} merge")
    if m.ref_q_off >= 0:  # the same queries also ran as one whole item on the GPU
        O, LSE = o.cpu().numpy(), lse.cpu().numpy()
        ref = slice(m.ref_q_off, m.ref_q_off + m.rows)
        hs = slice(m.head_begin, m.head_begin + m.head_cnt)
        assert np.abs(MO[:, hs] - O[ref, hs]).max() < 2e-2
        assert np.abs(ML[:, hs] - LSE[ref, hs]).max() < LSE_MAX_ABS


def test_merge_kernel_against_oracle_merge():
    from coalesced_attention_amd import zl
    rng = np.random.default_rng(3)
    # the last case is the largest part count the entry point accepts
    for d, n_parts, rows, H, h0, hc in [(128, 2, 300, 5, 1, 3), (64, 3, 77, 2, 0, 2), (128, 5, 16, 24, 4, 12),
                                        (64, 64, 7, 2, 0, 2)]:
        stride = rows + 9
        T = (n_parts - 1) * stride + rows + 4
        o = rng.standard_normal((T, H, d)).astype(np.float32)
        lse = (3 * rng.standard_normal((T, H))).astype(np.float32)
        lse[rng.random((T, H)) < 0.1] = -np.inf  # empty parts
        lse[4 + 5, :] = -np.inf
        lse[4 + stride + 5, :] = -np.inf  # row 5: every part empty when n_parts == 2
        if n_parts > 2:
            for p in range(2, n_parts):
                lse[4 + p * stride + 5, :] = -np.inf
        to = torch.from_numpy(o).cuda()
        tl = torch.from_numpy(lse).cuda()
        mo, ml = zl.merge_partials(to, tl, 4, n_parts, rows, stride, h0, hc)
        torch.cuda.synchronize()
        parts_o = np.stack([o[4 + p * stride:4 + p * stride + rows, h0:h0 + hc] for p in range(n_parts)])
        parts_l = np.stack([lse[4 + p * stride:4 + p * stride + rows, h0:h0 + hc] for p in range(n_parts)])
        ro, rl = orc.merge_partials(parts_o, parts_l)
        go, gl = mo.cpu().numpy()[:, h0:h0 + hc], ml.cpu().numpy()[:, h0:h0 + hc]
        np.testing.assert_allclose(go, ro, rtol=1e-5, atol=1e-5)
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
        fin = np.isfinite(rl)
        np.testing.assert_allclose(gl[fin], rl[fin], rtol=1e-6, atol=1e-5)
        assert np.all(go[5] == 0) and np.all(np.isneginf(gl[5]))


# ----------------------------------------------------------------- invariants

def test_bitwise_determinism_and_schedule_independence():
    wl = W.config(2)
    # a reduced mixed batch keeps this quick: the shard and 6 images
    items = wl.items[:1] + wl.items[1:4] + wl.items[25:28]
    inp = W.make_inputs(wl)
    q, k, v = to_device(inp)
    outs = []
    for n_slots in (256, 256, 0, 97, 1):
        _, o, lse = run_fwd(items, q, k, v, wl.num_heads, wl.head_dim, n_slots=n_slots)
        outs.append((o.cpu().numpy(), lse.cpu().numpy()))
    for o2, l2 in outs[1:]:
        assert np.array_equal(o2, outs[0][0], equal_nan=True)
        assert np.array_equal(l2, outs[0][1], equal_nan=True)


def test_key_split_bitwise_over_slot_counts_and_close_to_unsplit():
    """A split forward is bitwise the same for any slot count (every chunk is
    computed by one tile and merged in chunk order), and within rounding of
    the unsplit forward."""
    wl, inp, (q, k, v) = _workload(0)
    outs = []
    for n_slots in (256, 0, 7, 1):
        _, o, lse = run_fwd(wl.items, q, k, v, wl.num_heads, wl.head_dim, n_slots=n_slots, kv_chunk=64)
        outs.append((o.cpu().numpy(), lse.cpu().numpy()))
    for o2, l2 in outs[1:]:
        assert np.array_equal(o2, outs[0][0], equal_nan=True)
        assert np.array_equal(l2, outs[0][1], equal_nan=True)
    _, o, lse = run_fwd(wl.items, q, k, v, wl.num_heads, wl.head_dim)
    O, LSE = o.cpu().numpy(), lse.cpu().numpy()
    assert np.nanmax(np.abs(outs[0][0] - O)) < 5e-3
    assert np.nanmax(np.abs(outs[0][1] - LSE)) < 1e-5


def test_independence_across_packed_sequences():
    wl, inp, (q, k, v) = _workload(1)
    _, o1, l1 = run_fwd(wl.items, q, k, v, wl.num_heads, wl.head_dim)
    a = wl.items[5]
    k2, v2, q2 = k.clone(), v.clone(), q.clone()
    k2[a.kv_off:a.kv_off + a.kv_len] *= -2
    v2[a.kv_off:a.kv_off + a.kv_len] += 1
    q2[a.q_off:a.q_off + a.q_len] = 0
    _, o2, l2 = run_fwd(wl.items, q2, k2, v2, wl.num_heads, wl.head_dim)
    O1, O2, L1, L2 = (x.cpu().numpy() for x in (o1, o2, l1, l2))
    mask = np.ones(wl.q_rows, bool)
    mask[a.q_off:a.q_off + a.q_len] = False
    assert np.array_equal(O1[mask], O2[mask]) and np.array_equal(L1[mask], L2[mask])
    assert not np.allclose(O1[~mask], O2[~mask])


def test_isolated_launches_match_the_oracle_and_the_coalesced_launch():
    """The price table times items alone and per bucket (the per-(bucket,
    theta) prices whose sum the pages' planner takes as the step time). Each
    isolated launch is checked against the oracle on its own (every row of
    the images, sampled rows of every 128-row block of the shard, on every
    head); and since each (row, head) is computed by the same tile in the
    same key order either way, it also gives the coalesced launch's bits."""
    wl = W.config(2)
    items = wl.items[:1] + wl.items[1:3] + wl.items[25:27]
    inp = W.make_inputs(wl)
    q, k, v = to_device(inp)
    Qh, Kh, Vh = _host(inp.q), _host(inp.k), _host(inp.v)
    _, o, lse = run_fwd(items, q, k, v, wl.num_heads, wl.head_dim)
    O, LSE = o.cpu().numpy(), lse.cpu().numpy()
    for part in ([items[0]], items[1:2], items[1:3], items[3:4], items[3:]):
        _, o1, l1 = run_fwd(part, q, k, v, wl.num_heads, wl.head_dim)
        O1, L1 = o1.cpu().numpy(), l1.cpu().numpy()
        st = oracle_compare(Stats(), part, Qh, Kh, Vh, O1, L1, wl.softmax_scale, seed=41)
        st.assert_gates(f"isolated launch of {len(part)} item(s), q_len {part[0].q_len}")
        for it in part:
            rs = slice(it.q_off, it.q_off + it.q_len)
            assert np.array_equal(O1[rs], O[rs]) and np.array_equal(L1[rs], LSE[rs])


def test_closed_forms_on_gpu():
    H, d = 3, 128
    kv = 1000
    rng = np.random.default_rng(1)
    K = torch.from_numpy(rng.standard_normal((kv, H, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    V = torch.from_numpy(rng.standard_normal((kv, H, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    Q = torch.zeros((300, H, d), dtype=torch.bfloat16, device="cuda")
    items = [(0, 300, 0, kv, 0, H)]
    _, o, lse = run_fwd(items, Q, K, V, H, d)
    mean_v = V.float().mean(0)
    assert torch.allclose(o, mean_v.expand_as(o), atol=1e-5, rtol=0)
    assert torch.allclose(lse, torch.full_like(lse, math.log(kv)), atol=1e-5, rtol=0)
    Q = torch.from_numpy(rng.standard_normal((300, H, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    Vc = torch.full_like(V, -1.5)
    _, o, _ = run_fwd(items, Q, K, Vc, H, d)
    assert torch.allclose(o, torch.full_like(o, -1.5), atol=2e-3, rtol=0)
    # one key: O = v, LSE = scale * q.k
    _, o, lse = run_fwd([(0, 300, 7, 1, 0, H)], Q, K, V, H, d)
    assert torch.allclose(o, V[7].float().expand_as(o), atol=1e-5, rtol=1e-6)
    z = (Q.float() * K[7].float()).sum(-1) / math.sqrt(d)
    assert torch.allclose(lse, z, atol=1e-4, rtol=0)


@pytest.mark.parametrize("d", [64, 128])
def test_ragged_edges_and_head_splits(d):
    H = 4
    rng = np.random.default_rng(d)
    cases = [(1, 1), (1, 64), (255, 65), (256, 63), (257, 129), (300, 127), (31, 1000), (513, 256),
             (5, 0), (0, 10), (40, 2047)]
    items, q_off, kv_off = [], 0, 0
    for ql, kl in cases:
        items.append(W.Item(q_off, ql, kv_off, kl, 0, H))
        q_off += ql
        kv_off += kl
    # a head-split pair sharing query rows (Ulysses-style), different key ranges
    items.append(W.Item(q_off, 200, 0, 300, 0, 2))
    items.append(W.Item(q_off, 200, 300, 150, 2, 2))
    q_off += 200
    Q = rng.standard_normal((q_off, H, d)).astype(np.float32)
    K = rng.standard_normal((kv_off, H, d)).astype(np.float32)
    V = rng.standard_normal((kv_off, H, d)).astype(np.float32)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in (Q, K, V))
    for n_slots in (0, 7):
        _, o, lse = run_fwd(items, q.cuda(), k.cuda(), v.cuda(), H, d, n_slots=n_slots)
        O, L = o.cpu().numpy(), lse.cpu().numpy()
        st = Stats()
        for idx, it in enumerate(items):
            if it.q_len == 0:
                continue
            for h in range(it.head_begin, it.head_begin + it.head_cnt):
                rows = np.arange(it.q_len)
                o_ref, l_ref = orc.coalesced_forward_rows(q.float().numpy(), k.float().numpy(),
                                                          v.float().numpy(), it, h, rows, 1 / math.sqrt(d))
                if it.kv_len == 0:
                    assert np.all(O[it.q_off:it.q_off + it.q_len, h] == 0)
                    assert np.all(np.isneginf(L[it.q_off:it.q_off + it.q_len, h]))
                    continue
                st.add(idx, O[it.q_off + rows, h], o_ref, L[it.q_off + rows, h], l_ref)
        st.assert_gates(f"ragged d={d} n_slots={n_slots}")


def test_peaky_queries_exercise_the_running_max():
    wl = W.config(0)
    inp = W.make_inputs(wl, q_scale=4.0)
    q, k, v = to_device(inp)
    _, o, lse = run_fwd(wl.items, q, k, v, wl.num_heads, wl.head_dim)
    st = oracle_compare(Stats(), wl.items, _host(inp.q), _host(inp.k), _host(inp.v),
                        o.cpu().numpy(), lse.cpu().numpy(), wl.softmax_scale)
    st.assert_gates("config 0, queries x4")


@pytest.mark.parametrize("d", [64, 128])
def test_score_jumps_past_the_first_block_raise_the_shift(d):
    """Keys planted in later key blocks whose scores exceed the first block's
    maximum by about 60 (the running sums pass 2^32) and by over 128 (exp2
    would overflow in fp32), one of them in the ragged last block: the rows
    must be redone with a raised shift and still match the oracle."""
    H = 2
    items = [W.Item(0, 300, 0, 1000, 0, H)]
    g = torch.Generator().manual_seed(17)
    q = torch.randn((300, H, d), generator=g).to(torch.bfloat16)
    k = torch.randn((1000, H, d), generator=g)
    v = torch.randn((1000, H, d), generator=g).to(torch.bfloat16)
    c = math.log2(math.e) / math.sqrt(d)
    qf = q.float()
    k[400, 0] = 4.0 * qf[5, 0]       # block 6: about +60 in exp2 units for row 5
    k[700, 0] = 16.0 * qf[200, 0]    # block 10: past exp2's fp32 range for row 200
    k[999, 1] = 6.0 * qf[299, 1]     # last block (40 of 64 keys): row 299 of head 1
    k = k.to(torch.bfloat16)
    jump = float((qf[200, 0] * k[700, 0].float()).sum()) * c
    assert jump > 128, jump
    log(f"score jumps, d={d}: forward on GPU")
    _, o, lse = run_fwd(items, q.cuda(), k.cuda(), v.cuda(), H, d)
    st = oracle_compare(Stats(), items, _host(q), _host(k), _host(v), o.cpu().numpy(),
                        lse.cpu().numpy(), 1 / math.sqrt(d))
    st.assert_gates(f"score jumps, d={d}")


def test_scores_rising_along_the_keys_raise_the_shift_repeatedly():
    """Keys drift towards the direction of query row 0, so its scores (and
    those of rows correlated with it) climb by ~200 in exp2 units over 32
    key blocks: the running sums pass 2^32 every few blocks and the shift is
    raised again and again within one tile."""
    H, d = 1, 128
    items = [W.Item(0, 96, 0, 2000, 0, H)]
    g = torch.Generator().manual_seed(23)
    q = torch.randn((96, H, d), generator=g).to(torch.bfloat16)
    ramp = torch.linspace(0.0, 12.0, 2000).view(2000, 1, 1)
    k = (torch.randn((2000, H, d), generator=g) + ramp * q[0].float()).to(torch.bfloat16)
    v = torch.randn((2000, H, d), generator=g).to(torch.bfloat16)
    log("rising scores: forward on GPU")
    _, o, lse = run_fwd(items, q.cuda(), k.cuda(), v.cuda(), H, d)
    st = oracle_compare(Stats(), items, _host(q), _host(k), _host(v), o.cpu().numpy(),
                        lse.cpu().numpy(), 1 / math.sqrt(d))
    st.assert_gates("rising scores")


def test_binding_rejects_host_tensors_before_any_launch():
    """A host tensor among the outputs, gradients or merge buffers raises
    ValueError in the binding; no pointer of it reaches a kernel."""
    from coalesced_attention_amd import zl
    items = [W.Item(0, 64, 0, 64, 0, 2)]
    q, k, v = (torch.randn((64, 2, 64)).to(torch.bfloat16).cuda() for _ in range(3))
    wl = zl.build_worklist(items, 64, 64, 2, 64, n_slots=4, device=q.device)
    with pytest.raises(ValueError):
        zl.coalesced_attn_fwd(wl, q, k, v, o=torch.zeros((64, 2, 64)))
    with pytest.raises(ValueError):
        zl.coalesced_attn_fwd(wl, q, k.cpu(), v)
    o, lse = zl.coalesced_attn_fwd(wl, q, k, v)
    with pytest.raises(ValueError):
        zl.coalesced_attn_bwd(wl, q, k, v, o, lse, torch.zeros((64, 2, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        zl.coalesced_attn_bwd(wl, q, k, v, o, lse, q, dk=torch.zeros((64, 2, 64)))
    with pytest.raises(ValueError):
        zl.merge_partials(o, lse, 0, 2, 32, 32, 0, 2, o_out=torch.zeros((32, 2, 64)))
    with pytest.raises(ValueError):
        zl.merge_partials(o, lse, 0, 2, 32, 32, 0, 2,
                          o_out=torch.zeros((32, 2, 64), dtype=torch.float64, device=q.device))
    torch.cuda.synchronize()


def test_key_permutation_within_an_item():
    wl, inp, (q, k, v) = _workload(1)
    items = wl.items[:3]
    _, o1, l1 = run_fwd(items, q, k, v, wl.num_heads, wl.head_dim)
    a = items[1]
    perm = torch.randperm(a.kv_len, generator=torch.Generator().manual_seed(0)).cuda() + a.kv_off
    k2, v2 = k.clone(), v.clone()
    k2[a.kv_off:a.kv_off + a.kv_len] = k[perm]
    v2[a.kv_off:a.kv_off + a.kv_len] = v[perm]
    _, o2, l2 = run_fwd(items, q, k2, v2, wl.num_heads, wl.head_dim)
    sl = slice(a.q_off, a.q_off + a.q_len)
    assert (o1[sl] - o2[sl]).abs().max().item() < 2e-3
    assert (l1[sl] - l2[sl]).abs().max().item() < 1e-4


@pytest.mark.timeout(600)
def test_maximum_key_range_and_offsets_past_2gb():
    """One item with 2^20 keys on 8 heads (K and V are 2 GiB each, so key
    offsets in bytes pass 2^31) next to a short item placed after it; the
    forward must match the oracle on sampled rows of both."""
    H, d = 8, 128
    n_keys = 1 << 20
    items = [W.Item(0, 300, 0, n_keys, 0, H), W.Item(300, 40, n_keys, 70, 0, H)]
    g = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn((340, H, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((n_keys + 70, H, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((n_keys + 70, H, d), generator=g, device="cuda").to(torch.bfloat16)
    log("2^20-key item: forward on GPU")
    _, o, lse = run_fwd(items, q, k, v, H, d)
    O, LSE = o.cpu().numpy(), lse.cpu().numpy()
    Qh, Kh, Vh = (x.float().cpu().numpy() for x in (q, k, v))
    st = oracle_compare(Stats(), items, Qh, Kh, Vh, O, LSE, 1 / math.sqrt(d), full_limit=64,
                        seed=9)
    st.assert_gates("2^20-key item forward")


def test_uncovered_rows_and_empty_worklists_are_left_untouched():
    """Rows no item covers keep what the caller's buffers held; an empty
    worklist launches nothing, forward and backward."""
    from coalesced_attention_amd import zl
    H, d = 3, 128
    g = torch.Generator(device="cuda").manual_seed(21)
    q = torch.randn((300, H, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((200, H, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((200, H, d), generator=g, device="cuda").to(torch.bfloat16)
    sentinel = 7.25
    for items in ([], [W.Item(40, 100, 10, 150, 1, 2)]):
        wl = zl.build_worklist(items, 300, 200, H, d, device=q.device)
        o = torch.full((300, H, d), sentinel, device="cuda")
        lse = torch.full((300, H), sentinel, device="cuda")
        zl.coalesced_attn_fwd(wl, q, k, v, o, lse)
        dq, dk, dv = zl.coalesced_attn_bwd(wl, q, k, v, o, lse, q)
        torch.cuda.synchronize()
        covered = torch.zeros((300, H), dtype=torch.bool, device="cuda")
        for it in items:
            covered[it.q_off:it.q_off + it.q_len, it.head_begin:it.head_begin + it.head_cnt] = True
        assert torch.all(o[~covered] == sentinel) and torch.all(lse[~covered] == sentinel)
        assert torch.all(dq[~covered] == 0)
        if items:
            assert torch.isfinite(o[covered]).all() and torch.isfinite(lse[covered]).all()
        else:
            assert not dk.any() and not dv.any()

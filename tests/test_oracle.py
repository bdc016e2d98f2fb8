"""Pins of the fp64 oracle against things other than itself: hand-derived
closed forms, brute force without max shift, float64 library routines,
invariants that exact attention must satisfy, finite differences, and
planted mistakes that the pins must catch."""

import json
import math
import os

import numpy as np
import pytest
import torch

from coalesced_attention_amd import workloads as W
from oracle import attention as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _expr(s):
    if s == "-inf":
        return -math.inf
    return eval(s, {"ln": math.log})


@pytest.fixture(scope="module")
def cfg0():
    wl = W.config(0)
    inp = W.make_inputs(wl, keep_fp32=True)
    return wl, inp


# ------------------------------------------------------------ golden cases

def test_golden_attention_cases():
    data = json.load(open(GOLDEN))
    for case in data["attention"]:
        o, lse = orc.attention_rows(case["q"], case["k"], case["v"], case["scale"])
        np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-13, err_msg=case["name"])
        np.testing.assert_allclose(lse, [_expr(e) for e in case["lse_expr"]], rtol=0, atol=1e-13,
                                   err_msg=case["name"])


def test_golden_merge_cases():
    data = json.load(open(GOLDEN))
    for case in data["merge"]:
        lse_parts = [[_expr(e) for e in p] for p in case["lse_parts_expr"]]
        o, lse = orc.merge_partials(case["o_parts"], lse_parts)
        np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-14, err_msg=case["name"])
        exp_lse = [_expr(e) for e in case["lse_expr"]]
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(exp_lse))
        fin = ~np.isneginf(np.asarray(exp_lse))
        np.testing.assert_allclose(np.asarray(lse)[fin], np.asarray(exp_lse)[fin], atol=1e-14)


# ------------------------------------------------------------ brute force

def _brute_check(fwd, wl, inp, rows_per_item=None):
    """Compare ``fwd`` (an attention_rows-like callable) with the pure-Python
    brute force on the unrounded fp32 draws of the tiny workload."""
    Q, K, V = inp.q32.astype(np.float64), inp.k32.astype(np.float64), inp.v32.astype(np.float64)
    s = wl.softmax_scale
    worst = 0.0
    rng = np.random.default_rng(11)
    for it in wl.items:
        rows = np.arange(it.q_len) if (rows_per_item is None or it.q_len <= rows_per_item) \
            else np.sort(rng.choice(it.q_len, rows_per_item, replace=False))
        for h in range(it.head_begin, it.head_begin + it.head_cnt):
            k = K[it.kv_off:it.kv_off + it.kv_len, h]
            v = V[it.kv_off:it.kv_off + it.kv_len, h]
            o, lse = fwd(Q[it.q_off + rows, h], k, v, s)
            kl, vl = k.tolist(), v.tolist()
            for i, r in enumerate(rows):
                bo, blse = orc.brute_attention_row(Q[it.q_off + r, h].tolist(), kl, vl, s)
                worst = max(worst, np.max(np.abs(np.asarray(bo) - o[i])) / max(1.0, np.max(np.abs(bo))))
                worst = max(worst, abs(blse - lse[i]) / max(1.0, abs(blse)))
    return worst


def test_oracle_matches_brute_force(cfg0):
    wl, inp = cfg0
    assert _brute_check(orc.attention_rows, wl, inp, rows_per_item=40) < 1e-12


def test_oracle_matches_sdpa_and_logsumexp_float64(cfg0):
    wl, inp = cfg0
    Q, K, V = (torch.from_numpy(x.astype(np.float64)) for x in (inp.q32, inp.k32, inp.v32))
    s = wl.softmax_scale
    O, LSE = orc.coalesced_forward(inp.q32, inp.k32, inp.v32, wl.items, s)
    for it in wl.items:
        q = Q[it.q_off:it.q_off + it.q_len].transpose(0, 1)  # [H, r, d]
        k = K[it.kv_off:it.kv_off + it.kv_len].transpose(0, 1)
        v = V[it.kv_off:it.kv_off + it.kv_len].transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=s)
        ref_lse = torch.logsumexp(s * q @ k.transpose(1, 2), dim=-1)
        np.testing.assert_allclose(O[it.q_off:it.q_off + it.q_len].transpose(1, 0, 2), ref.numpy(),
                                   rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(LSE[it.q_off:it.q_off + it.q_len].T, ref_lse.numpy(),
                                   rtol=1e-13, atol=1e-13)


def test_coverage_marks_uncovered_rows_nan():
    Q = np.zeros((10, 2, 4)); K = np.ones((6, 2, 4)); V = np.ones((6, 2, 4))
    O, LSE = orc.coalesced_forward(Q, K, V, [(0, 4, 0, 3, 1, 1), (6, 2, 3, 3, 0, 2)], 0.5)
    covered = np.zeros((10, 2), bool)
    covered[0:4, 1] = True
    covered[6:8, :] = True
    assert np.array_equal(~np.isnan(LSE), covered)
    assert np.array_equal(~np.isnan(O).any(-1), covered)


# ------------------------------------------------------------ closed forms

def test_closed_forms():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((37, 16)); v = rng.standard_normal((37, 16))
    # zero queries: uniform weights
    o, lse = orc.attention_rows(np.zeros((3, 16)), k, v, 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, np.log(37), atol=1e-14)
    # one key: O = v, LSE = z
    q = rng.standard_normal((5, 16))
    o, lse = orc.attention_rows(q, k[:1], v[:1], 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(v[0], o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, 0.25 * q @ k[0], atol=1e-13)
    # constant values: O = c
    o, _ = orc.attention_rows(q, k, np.full((37, 16), -1.75), 0.25)
    np.testing.assert_allclose(o, -1.75, atol=1e-14)
    # no keys
    o, lse = orc.attention_rows(q, k[:0], v[:0], 0.25)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_peaky_scores_stay_finite():
    # scores of several hundred: only the max-shifted form stays finite
    rng = np.random.default_rng(5)
    q = 40 * rng.standard_normal((4, 64)); k = rng.standard_normal((50, 64)); v = rng.standard_normal((50, 64))
    o, lse = orc.attention_rows(q, k, v, 1 / 8)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    z = q @ k.T / 8
    j = z.argmax(1)
    # at these gaps softmax is nearly one-hot
    gap = np.sort(z, 1)[:, -1] - np.sort(z, 1)[:, -2]
    for r in range(4):
        if gap[r] > 40:
            np.testing.assert_allclose(o[r], v[j[r]], atol=1e-12)


# ------------------------------------------------------------ invariants

def test_invariants(cfg0):
    wl, inp = cfg0
    Q, K, V = (x.astype(np.float64) for x in (inp.q32, inp.k32, inp.v32))
    s = wl.softmax_scale
    it = wl.items[2]
    h = 1
    q = Q[it.q_off:it.q_off + it.q_len, h]; k = K[it.kv_off:it.kv_off + it.kv_len, h]
    v = V[it.kv_off:it.kv_off + it.kv_len, h]
    o, lse = orc.attention_rows(q, k, v, s)
    rng = np.random.default_rng(9)
    perm = rng.permutation(len(k))
    o2, lse2 = orc.attention_rows(q, k[perm], v[perm], s)
    np.testing.assert_allclose(o2, o, atol=1e-13); np.testing.assert_allclose(lse2, lse, atol=1e-13)
    qp = rng.permutation(len(q))
    o3, lse3 = orc.attention_rows(q[qp], k, v, s)
    np.testing.assert_allclose(o3, o[qp], atol=1e-14); np.testing.assert_allclose(lse3, lse[qp], atol=1e-14)
    u = rng.standard_normal(k.shape[1])
    o4, lse4 = orc.attention_rows(q, k + u, v, s)
    np.testing.assert_allclose(o4, o, atol=1e-12)
    np.testing.assert_allclose(lse4, lse + s * q @ u, atol=1e-12)
    o5, lse5 = orc.attention_rows(q, k, -2.5 * v + 0.75, s)
    np.testing.assert_allclose(o5, -2.5 * o + 0.75, atol=1e-12); np.testing.assert_allclose(lse5, lse, atol=0)


def test_independence_across_packed_sequences(cfg0):
    wl, inp = cfg0
    Q, K, V = (x.astype(np.float64) for x in (inp.q32, inp.k32, inp.v32))
    O, LSE = orc.coalesced_forward(Q, K, V, wl.items, wl.softmax_scale)
    K2, V2, Q2 = K.copy(), V.copy(), Q.copy()
    a = wl.items[0]
    K2[a.kv_off:a.kv_off + a.kv_len] += 3.0
    V2[a.kv_off:a.kv_off + a.kv_len] *= -1.0
    Q2[a.q_off:a.q_off + a.q_len] = 0.0
    O2, LSE2 = orc.coalesced_forward(Q2, K2, V2, wl.items, wl.softmax_scale)
    rest = slice(a.q_len, wl.q_rows)
    assert np.array_equal(O2[rest], O[rest]) and np.array_equal(LSE2[rest], LSE[rest])
    assert not np.allclose(O2[:a.q_len], O[:a.q_len])


# ------------------------------------------------------------ merge

def test_merge_of_kv_split_equals_whole(cfg0):
    wl, inp = cfg0
    s = wl.softmax_scale
    O, LSE = orc.coalesced_forward(inp.q32, inp.k32, inp.v32, wl.items, s)
    m = wl.merges[0]
    parts_o = np.stack([O[m.row0 + p * m.part_row_stride:m.row0 + p * m.part_row_stride + m.rows]
                        for p in range(m.n_parts)])
    parts_l = np.stack([LSE[m.row0 + p * m.part_row_stride:m.row0 + p * m.part_row_stride + m.rows]
                        for p in range(m.n_parts)])
    mo, ml = orc.merge_partials(parts_o, parts_l)
    ref = slice(m.ref_q_off, m.ref_q_off + m.rows)
    np.testing.assert_allclose(mo, O[ref], atol=1e-13)
    np.testing.assert_allclose(ml, LSE[ref], atol=1e-13)


def test_merge_three_uneven_splits_and_identities():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((9, 32)); k = rng.standard_normal((101, 32)); v = rng.standard_normal((101, 32))
    o, lse = orc.attention_rows(q, k, v, 0.3)
    cuts = [0, 17, 18, 101]  # a one-key part, a long part
    parts = [orc.attention_rows(q, k[a:b], v[a:b], 0.3) for a, b in zip(cuts, cuts[1:])]
    mo, ml = orc.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(mo, o, atol=1e-13); np.testing.assert_allclose(ml, lse, atol=1e-13)
    # two identical parts: O unchanged, LSE + ln 2
    mo, ml = orc.merge_partials(np.stack([o, o]), np.stack([lse, lse]))
    np.testing.assert_allclose(mo, o, atol=1e-14); np.testing.assert_allclose(ml, lse + math.log(2), atol=1e-14)
    # an empty part returns the other
    empty_o, empty_l = orc.attention_rows(q, k[:0], v[:0], 0.3)
    mo, ml = orc.merge_partials(np.stack([empty_o, o]), np.stack([empty_l, lse]))
    np.testing.assert_allclose(mo, o, atol=0); np.testing.assert_allclose(ml, lse, atol=0)


# ------------------------------------------------------------ backward

def _fd_check(bwd, wl, inp, n_coords=256, seed=4):
    """Max over sampled coordinates of |central difference - VJP| relative to
    max(1, |VJP|) for F = sum(dO * O), on the tiny workload in fp64."""
    Q, K, V = (x.astype(np.float64) for x in (inp.q32, inp.k32, inp.v32))
    dO = inp.dout.double().numpy()
    s = wl.softmax_scale
    dQ, dK, dV = bwd(Q, K, V, dO, wl.items, s)

    def F(Qx, Kx, Vx):
        O, _ = orc.coalesced_forward(Qx, Kx, Vx, wl.items, s)
        return np.nansum(dO * np.nan_to_num(O))

    rng = np.random.default_rng(seed)
    worst = 0.0
    for name, X, G in (("q", Q, dQ), ("k", K, dK), ("v", V, dV)):
        flat = rng.choice(X.size, n_coords, replace=False)
        for f in flat:
            idx = np.unravel_index(f, X.shape)
            x0 = X[idx]
            hstep = 1e-6 * max(1.0, abs(x0))
            args = [Q, K, V]
            Xp = X.copy(); Xp[idx] = x0 + hstep
            Xm = X.copy(); Xm[idx] = x0 - hstep
            ip = {"q": 0, "k": 1, "v": 2}[name]
            ap = list(args); ap[ip] = Xp
            am = list(args); am[ip] = Xm
            fd = (F(*ap) - F(*am)) / (2 * hstep)
            worst = max(worst, abs(fd - G[idx]) / max(1.0, abs(G[idx])))
    return worst


@pytest.mark.slow
def test_backward_finite_differences(cfg0):
    wl, inp = cfg0
    assert _fd_check(orc.coalesced_backward, wl, inp, n_coords=256) < 1e-6


def test_backward_matches_autograd_float64(cfg0):
    wl, inp = cfg0
    s = wl.softmax_scale
    Q, K, V = (x.astype(np.float64) for x in (inp.q32, inp.k32, inp.v32))
    dO = inp.dout.double().numpy()
    dQ, dK, dV = orc.coalesced_backward(Q, K, V, dO, wl.items, s)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    total = 0
    for it in wl.items:
        q = tq[it.q_off:it.q_off + it.q_len].transpose(0, 1)
        k = tk[it.kv_off:it.kv_off + it.kv_len].transpose(0, 1)
        v = tv[it.kv_off:it.kv_off + it.kv_len].transpose(0, 1)
        o = torch.softmax(s * q @ k.transpose(1, 2), -1) @ v
        total = total + (o * torch.from_numpy(dO[it.q_off:it.q_off + it.q_len]).transpose(0, 1)).sum()
    total.backward()
    np.testing.assert_allclose(dQ, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), atol=1e-12)


def test_backward_identities(cfg0):
    wl, inp = cfg0
    s = wl.softmax_scale
    Q, K, V = (x.astype(np.float64) for x in (inp.q32, inp.k32, inp.v32))
    dO = inp.dout.double().numpy()
    it = wl.items[1]
    for h in range(2):
        args = (Q[it.q_off:it.q_off + it.q_len, h], K[it.kv_off:it.kv_off + it.kv_len, h],
                V[it.kv_off:it.kv_off + it.kv_len, h], dO[it.q_off:it.q_off + it.q_len, h])
        dq, dk, dv, o, lse = orc.attention_backward_item(*args, s)
        np.testing.assert_allclose(dk.sum(0), 0, atol=1e-11)  # sum_j dS_rj = 0
        np.testing.assert_allclose(dv.sum(0), args[3].sum(0), atol=1e-11)  # rows of P sum to 1
        dq0, dk0, dv0, _, _ = orc.attention_backward_item(args[0], args[1], np.full_like(args[2], 0.5), args[3], s)
        assert np.abs(dq0).max() < 1e-12 and np.abs(dk0).max() < 1e-12


# ------------------------------------------------------------ planted mistakes

def _mutant_no_scale(q, k, v, scale):
    return orc.attention_rows(q, k, v, 1.0)


def _mutant_log2_lse(q, k, v, scale):
    o, lse = orc.attention_rows(q, k, v, scale)
    return o, lse / math.log(2)


def _mutant_transposed_values(q, k, v, scale):
    # values taken in reverse key order: a wrong index on V
    return orc.attention_rows(q, k, v[::-1], scale)


def _mutant_max_not_added(q, k, v, scale):
    q64, k64 = np.asarray(q, float), np.asarray(k, float)
    z = scale * q64 @ k64.T
    o, lse = orc.attention_rows(q, k, v, scale)
    return o, lse - z.max(1)


@pytest.mark.parametrize("mutant", [_mutant_no_scale, _mutant_log2_lse, _mutant_transposed_values,
                                    _mutant_max_not_added])
def test_brute_force_pin_catches_planted_forward_mistakes(cfg0, mutant):
    wl, inp = cfg0
    assert _brute_check(mutant, wl, inp, rows_per_item=4) > 1e-6


def test_merge_golden_pin_catches_unnormalised_weights():
    data = json.load(open(GOLDEN))
    case = data["merge"][0]
    lse_parts = np.array([[_expr(e) for e in p] for p in case["lse_parts_expr"]])
    o_parts = np.asarray(case["o_parts"])
    w = np.exp(lse_parts - lse_parts.max(0))  # planted: forgot to divide by the sum
    bad = (w[..., None] * o_parts).sum(0)
    assert not np.allclose(bad, case["o"], atol=1e-3)


def _bwd_mutant_sign(Q, K, V, dO, items, s):
    dQ, dK, dV = orc.coalesced_backward(Q, K, V, dO, items, s)
    # planted: dS = P * (dP + D) changes dQ and dK; emulate by recomputing
    dQm, dKm = np.zeros_like(dQ), np.zeros_like(dK)
    for it in items:
        for h in range(it.head_begin, it.head_begin + it.head_cnt):
            q = Q[it.q_off:it.q_off + it.q_len, h]; k = K[it.kv_off:it.kv_off + it.kv_len, h]
            v = V[it.kv_off:it.kv_off + it.kv_len, h]; do = dO[it.q_off:it.q_off + it.q_len, h]
            z = s * q @ k.T
            p = np.exp(z - z.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
            D = (do * (p @ v)).sum(1)
            ds = p * (do @ v.T + D[:, None])
            dQm[it.q_off:it.q_off + it.q_len, h] += s * ds @ k
            dKm[it.kv_off:it.kv_off + it.kv_len, h] += s * ds.T @ q
    return dQm, dKm, dV


def _bwd_mutant_no_scale(Q, K, V, dO, items, s):
    dQ, dK, dV = orc.coalesced_backward(Q, K, V, dO, items, s)
    return dQ / s, dK, dV


def _bwd_mutant_dv_transposed_rows(Q, K, V, dO, items, s):
    dQ, dK, dV = orc.coalesced_backward(Q, K, V, dO, items, s)
    return dQ, dK, dV[::-1]


@pytest.mark.parametrize("mutant", [_bwd_mutant_sign, _bwd_mutant_no_scale, _bwd_mutant_dv_transposed_rows])
def test_finite_difference_pin_catches_planted_backward_mistakes(cfg0, mutant):
    wl, inp = cfg0
    assert _fd_check(mutant, wl, inp, n_coords=24, seed=8) > 1e-3


# ------------------------------------------------------------ sampled forms
#
# The full-size GPU checks go through two sampled forms of the oracle:
# coalesced_forward_rows (chosen query rows of one item and head) and
# attention_backward_sampled (dQ at chosen rows, dK / dV at chosen keys).
# Both are pinned here at packed offsets and head ranges that do not start
# at zero, where an indexing slip (rows taken from 0 instead of q_off, keys
# without kv_off, the wrong head) would show.

def _packed_case(seed=31, H=4, d=16):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((300, H, d))
    K = rng.standard_normal((260, H, d))
    V = rng.standard_normal((260, H, d))
    dO = rng.standard_normal((300, H, d))
    items = [W.Item(37, 90, 21, 150, 1, 2),    # offsets and heads away from 0
             W.Item(127, 130, 171, 89, 3, 1),  # last head only
             W.Item(0, 37, 0, 21, 0, 4)]
    return Q, K, V, dO, items


def _rows_check(fn, Q, K, V, items, scale, seed=2):
    """Largest error of fn (a coalesced_forward_rows-like callable) against
    the pure-Python brute force at explicit packed indices."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for it in items:
        rows = np.sort(rng.choice(it.q_len, min(it.q_len, 6), replace=False))
        for h in range(it.head_begin, it.head_begin + it.head_cnt):
            o, lse = fn(Q, K, V, it, h, rows, scale)
            kl = K[it.kv_off:it.kv_off + it.kv_len, h].tolist()
            vl = V[it.kv_off:it.kv_off + it.kv_len, h].tolist()
            for i, r in enumerate(rows):
                bo, blse = orc.brute_attention_row(Q[it.q_off + r, h].tolist(), kl, vl, scale)
                worst = max(worst, float(np.abs(np.asarray(bo) - o[i]).max()), abs(blse - lse[i]))
    return worst


def test_forward_rows_at_packed_offsets_match_brute_force_and_full_forward(cfg0):
    Q, K, V, _, items = _packed_case()
    assert _rows_check(orc.coalesced_forward_rows, Q, K, V, items, 0.25) < 1e-12
    wl, inp = cfg0
    Qc, Kc, Vc = (x.astype(np.float64) for x in (inp.q32, inp.k32, inp.v32))
    assert _rows_check(orc.coalesced_forward_rows, Qc, Kc, Vc, wl.items, wl.softmax_scale) < 1e-12
    # and the full coalesced forward at the same packed rows
    O, LSE = orc.coalesced_forward(Q, K, V, items, 0.25)
    for it in items:
        rows = np.arange(0, it.q_len, 7)
        for h in range(it.head_begin, it.head_begin + it.head_cnt):
            o, lse = orc.coalesced_forward_rows(Q, K, V, it, h, rows, 0.25)
            np.testing.assert_allclose(o, O[it.q_off + rows, h], atol=1e-13)
            np.testing.assert_allclose(lse, LSE[it.q_off + rows, h], atol=1e-13)


def _rows_mutant_rows_from_zero(Q, K, V, it, h, rows, scale):
    return orc.attention_rows(Q[rows, h], K[it.kv_off:it.kv_off + it.kv_len, h],
                              V[it.kv_off:it.kv_off + it.kv_len, h], scale)


def _rows_mutant_keys_from_zero(Q, K, V, it, h, rows, scale):
    return orc.attention_rows(Q[it.q_off + rows, h], K[:it.kv_len, h], V[:it.kv_len, h], scale)


def _rows_mutant_head_within_item(Q, K, V, it, h, rows, scale):
    hh = h - it.head_begin  # head index taken relative to the item
    return orc.attention_rows(Q[it.q_off + rows, hh], K[it.kv_off:it.kv_off + it.kv_len, hh],
                              V[it.kv_off:it.kv_off + it.kv_len, hh], scale)


@pytest.mark.parametrize("mutant", [_rows_mutant_rows_from_zero, _rows_mutant_keys_from_zero,
                                    _rows_mutant_head_within_item])
def test_forward_rows_pin_catches_planted_indexing_mistakes(mutant):
    Q, K, V, _, items = _packed_case()
    assert _rows_check(mutant, Q, K, V, items, 0.25) > 1e-3


def _sampled_check(fn, Q, K, V, dO, items, scale, chunk, seed=3):
    """Largest error of fn (an attention_backward_sampled-like callable)
    against the full-matrix backward at seeded rows and keys of every item
    and head (all of them for the short items)."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for it in items:
        rows = np.arange(it.q_len) if it.q_len <= 40 else np.sort(rng.choice(it.q_len, 9, replace=False))
        cols = np.arange(it.kv_len) if it.kv_len <= 40 else np.sort(rng.choice(it.kv_len, 11, replace=False))
        for h in range(it.head_begin, it.head_begin + it.head_cnt):
            args = (Q[it.q_off:it.q_off + it.q_len, h], K[it.kv_off:it.kv_off + it.kv_len, h],
                    V[it.kv_off:it.kv_off + it.kv_len, h], dO[it.q_off:it.q_off + it.q_len, h])
            rq, rk, rv, _, _ = orc.attention_backward_item(*args, scale)
            dq, dk, dv = fn(*args, scale, rows, cols, chunk=chunk)
            worst = max(worst, float(np.abs(dq - rq[rows]).max(initial=0)),
                        float(np.abs(dk - rk[cols]).max(initial=0)),
                        float(np.abs(dv - rv[cols]).max(initial=0)))
    return worst


@pytest.mark.parametrize("chunk", [512, 37, 1])
def test_backward_sampled_matches_full_matrix_backward(cfg0, chunk):
    """Row chunks of 37 and 1 cut every item mid-way, so LSE, D and the key
    sums have to be carried across chunks correctly."""
    Q, K, V, dO, items = _packed_case()
    assert _sampled_check(orc.attention_backward_sampled, Q, K, V, dO, items, 0.25, chunk) < 1e-12
    wl, inp = cfg0
    Qc, Kc, Vc = (x.astype(np.float64) for x in (inp.q32, inp.k32, inp.v32))
    dOc = inp.dout.double().numpy()
    assert _sampled_check(orc.attention_backward_sampled, Qc, Kc, Vc, dOc, wl.items,
                          wl.softmax_scale, chunk) < 1e-12


def test_backward_sampled_all_positions_equal_the_coalesced_backward(cfg0):
    wl, inp = cfg0
    Q, K, V = (x.astype(np.float64) for x in (inp.q32, inp.k32, inp.v32))
    dO = inp.dout.double().numpy()
    s = wl.softmax_scale
    it = wl.items[2]
    dQ, dK, dV = orc.coalesced_backward(Q, K, V, dO, [it], s)
    for h in range(2):
        dq, dk, dv = orc.attention_backward_sampled(
            Q[it.q_off:it.q_off + it.q_len, h], K[it.kv_off:it.kv_off + it.kv_len, h],
            V[it.kv_off:it.kv_off + it.kv_len, h], dO[it.q_off:it.q_off + it.q_len, h], s,
            np.arange(it.q_len), np.arange(it.kv_len), chunk=64)
        np.testing.assert_allclose(dq, dQ[it.q_off:it.q_off + it.q_len, h], atol=1e-12)
        np.testing.assert_allclose(dk, dK[it.kv_off:it.kv_off + it.kv_len, h], atol=1e-12)
        np.testing.assert_allclose(dv, dV[it.kv_off:it.kv_off + it.kv_len, h], atol=1e-12)
        np.testing.assert_allclose(dk.sum(0), 0, atol=1e-11)  # sum_j dS_rj = 0


def _sampled_mutant_lse_over_sampled_keys(q, k, v, do, scale, rows, cols, chunk=512):
    # planted: the softmax normalised over the sampled keys only
    k, v = np.asarray(k)[cols], np.asarray(v)[cols]
    return orc.attention_backward_sampled(q, k, v, do, scale, rows, np.arange(len(cols)), chunk=chunk)


def _sampled_mutant_key_sums_over_sampled_rows(q, k, v, do, scale, rows, cols, chunk=512):
    # planted: dK / dV summed over the sampled query rows only
    dq, _, _ = orc.attention_backward_sampled(q, k, v, do, scale, rows, cols, chunk=chunk)
    full = orc.attention_backward_item(q, k, v, do, scale)
    z = scale * (np.asarray(q)[rows] @ np.asarray(k).T)
    p = np.exp(z - full[4][rows, None])
    ds = p * (np.asarray(do)[rows] @ np.asarray(v).T - (np.asarray(do)[rows] * full[3][rows]).sum(1)[:, None])
    return dq, scale * (ds[:, cols].T @ np.asarray(q)[rows]), p[:, cols].T @ np.asarray(do)[rows]


def _sampled_mutant_last_chunk_only(q, k, v, do, scale, rows, cols, chunk=512):
    # planted: key sums reset at every chunk instead of accumulated
    n = np.asarray(q).shape[0]
    start = (n - 1) // chunk * chunk
    dq, _, _ = orc.attention_backward_sampled(q, k, v, do, scale, rows, cols, chunk=chunk)
    _, dk, dv = orc.attention_backward_sampled(np.asarray(q)[start:], k, v, np.asarray(do)[start:], scale,
                                               np.zeros(0, np.int64), cols, chunk=chunk)
    return dq, dk, dv


@pytest.mark.parametrize("mutant", [_sampled_mutant_lse_over_sampled_keys,
                                    _sampled_mutant_key_sums_over_sampled_rows,
                                    _sampled_mutant_last_chunk_only])
def test_backward_sampled_pin_catches_planted_mistakes(mutant):
    Q, K, V, dO, items = _packed_case()
    assert _sampled_check(mutant, Q, K, V, dO, items, 0.25, chunk=37) > 1e-3

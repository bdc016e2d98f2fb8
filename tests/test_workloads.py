"""The synthetic workloads: shapes, theta expansion and seeded draws."""

import numpy as np
import pytest

from coalesced_attention_amd import workloads as W
from oracle.worklist import cut_tiles


def test_theta_expansion_tiles_the_sequence():
    # every rank's share together covers each (query, head, key) triple once
    L, H = 1003, 6
    for theta in [(1, 1, 1), (4, 1, 1), (1, 2, 1), (1, 1, 3), (3, 2, 2)]:
        q, h, k = theta
        cover = np.zeros((L, H, L), np.int8)
        qstart = 0
        for iq in range(q):
            for ih in range(h):
                for ik in range(k):
                    it = W.theta_item(L, H, theta, (iq, ih, ik), q_off=0, kv_base=0)
                    s, n = W.split_bounds(L, q, iq)
                    assert n == it.q_len
                    cover[s:s + n, it.head_begin:it.head_begin + it.head_cnt,
                          it.kv_off:it.kv_off + it.kv_len] += 1
        assert cover.min() == 1 and cover.max() == 1, theta
    assert W.theta_item(100, 24, (1, 1, 1), (0, 0, 0), 7, 9) == W.Item(7, 100, 9, 100, 0, 24)


def test_theta_legality():
    with pytest.raises(ValueError):
        W.theta_item(100, 24, (1, 5, 1), (0, 0, 0), 0, 0)  # 5 does not divide 24
    with pytest.raises(ValueError):
        W.theta_item(100, 24, (2, 1, 1), (2, 0, 0), 0, 0)


EXPECTED = {  # (q_rows, kv_rows, n_items, tiles at 128 rows, forward flops)
    0: (932, 420, 5, 16, None),
    1: (36864, 36864, 48, 6912, 4.252e11),
    2: (40958, 65528, 57, 7680, 3.632e12),
    3: (71284, 235984, 18, 8232, 3.724e13),
    4: (40958, 65528, 57, 7680, 3.632e12),
    # 36900 x 147600 x 24 heads + 13 x 1024^2 x 24, and 41820 x 334560 x 12 + 8 x 1024^2 x 24
    5: (50212, 160912, 14, 289 * 24 + 13 * 8 * 24, 4 * 128 * (36900 * 147600 * 24 + 13 * 1024 ** 2 * 24)),
    6: (50012, 342752, 9, 327 * 12 + 8 * 8 * 24, 4 * 128 * (41820 * 334560 * 12 + 8 * 1024 ** 2 * 24)),
}


@pytest.mark.parametrize("c", range(W.NUM_CONFIGS))
def test_config_shapes(c):
    wl = W.config(c)
    qr, kr, n, tiles, flops = EXPECTED[c]
    assert (wl.q_rows, wl.kv_rows, len(wl.items)) == (qr, kr, n)
    assert len(cut_tiles(wl.items, 128, 0)) == tiles
    if flops:
        assert abs(wl.flops_fwd() / flops - 1) < 1e-3
    # items stay inside the buffers and never write the same (row, head) twice
    cov = np.zeros((wl.q_rows, wl.num_heads), np.int32)
    for it in wl.items:
        assert 0 <= it.q_off and it.q_off + it.q_len <= wl.q_rows
        assert 0 <= it.kv_off and it.kv_off + it.kv_len <= wl.kv_rows
        assert 0 <= it.head_begin and it.head_begin + it.head_cnt <= wl.num_heads
        cov[it.q_off:it.q_off + it.q_len, it.head_begin:it.head_begin + it.head_cnt] += 1
    assert cov.max() == 1


def test_config0_layout_matches_appendix():
    wl = W.config(0)
    assert [it.as_tuple() for it in wl.items] == [
        (0, 64, 0, 64, 0, 2), (64, 100, 64, 100, 0, 2), (164, 256, 164, 256, 0, 2),
        (420, 256, 164, 128, 0, 2), (676, 256, 292, 128, 0, 2)]


def test_draws_are_seeded_and_chunk_independent():
    a = W.draw_normal(5, W.TENSOR_K, 5000, (2, 3))
    b = W.draw_normal(5, W.TENSOR_K, 5000, (2, 3))
    assert np.array_equal(a, b)
    c = W.draw_normal(5, W.TENSOR_K, 1500, (2, 3), row_start=3000)
    assert np.array_equal(a[3000:4500], c)
    assert not np.array_equal(a, W.draw_normal(5, W.TENSOR_V, 5000, (2, 3)))
    assert abs(a.mean()) < 0.05 and abs(a.std() - 1) < 0.05


def test_make_inputs_copies_and_rounding():
    wl = W.config(0)
    inp = W.make_inputs(wl, keep_fp32=True)
    assert inp.q.shape == (932, 2, 64) and inp.k.shape == (420, 2, 64)
    assert np.array_equal(inp.q32[420:676], inp.q32[164:420])
    assert np.array_equal(inp.q32[676:932], inp.q32[164:420])
    # bf16 keeps 8 significant bits: round to nearest even errs by at most 2^-8 |x|
    err = np.abs(inp.q.float().numpy() - inp.q32)
    assert np.all(err <= np.abs(inp.q32) * 2.0 ** -8 + 1e-30)


def test_sample_rows_cover_every_block():
    it = W.Item(0, 8190, 0, 32760, 0, 24)
    rows = W.sample_rows(it, seed=1)
    blocks = set(rows // 128)
    assert blocks == set(range((8190 + 127) // 128))
    assert rows[0] == 0 and rows[-1] == 8189
    small = W.Item(0, 1024, 0, 1024, 0, 24)
    assert len(W.sample_rows(small, seed=1)) == 1024

"""The C-ABI library on the CPU: it loads, exports what include/*.h declare,
its worklist equals the reference LPT schedule bit for bit, and every
argument error is rejected on the host before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

from coalesced_attention_amd import workloads as W
from coalesced_attention_amd import zl
from oracle.worklist import lpt_schedule, lpt_schedule_bwd, split_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zl.h")
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(zl_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == set(zl.EXPORTS)
    for name in declared:
        assert hasattr(zl.lib, name), name


def test_abi_version_and_status_strings():
    text = open(HEADER).read()
    assert zl.ABI_VERSION == int(re.search(r"#define ZL_ABI_VERSION (\d+)", text).group(1))
    for code in zl.STATUS:
        assert zl.lib.zl_status_string(code)
    assert zl.lib.zl_status_string(-1234) == b"unknown status"


@pytest.mark.parametrize("cfg,n_slots", [(0, 0), (0, 3), (1, 256), (2, 0), (2, 256), (2, 97), (3, 256),
                                         (3, 1)])
def test_worklist_matches_reference_schedule(cfg, n_slots):
    wl = W.config(cfg)
    built = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim,
                              n_slots=n_slots)
    h = built.header
    assert h.magic == zl.WORKLIST_MAGIC and h.abi_version == zl.ABI_VERSION
    assert (h.q_rows, h.kv_rows, h.num_heads, h.head_dim) == (wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim)
    assert h.softmax_scale == np.float32(1 / np.sqrt(wl.head_dim))
    ref, begin, loads = lpt_schedule(wl.items, h.block_m, n_slots, h.cost_c0)
    got = built.tiles()
    assert h.n_tiles == len(ref) == len(got)
    want = np.array([(t.q_row0, t.kv_row0, t.q_rows, t.kv_len, t.head, t.item) for t in ref], dtype=zl.TILE_DTYPE)
    assert np.array_equal(got, want)
    if n_slots:
        assert list(built.slots()) == begin
        assert h.max_slot_cost == max(loads)
    assert h.total_cost == sum(t.cost for t in ref)
    # backward: key blocks x heads x items, same LPT rule
    c0_bwd = h.block_n_bwd * (h.cost_c0 // h.block_m)
    bref, bbegin, bloads = lpt_schedule_bwd(wl.items, h.block_n_bwd, n_slots, c0_bwd)
    bgot = built.bwd_tiles()
    assert h.n_bwd_tiles == len(bref) == len(bgot)
    bwant = np.array([(t.q_row0, t.kv_row0, t.q_rows, t.kv_len, t.head, t.item) for t in bref],
                     dtype=zl.TILE_DTYPE)
    assert np.array_equal(bgot, bwant)
    if n_slots:
        assert list(built.bwd_slots()) == bbegin and h.bwd_max_slot_cost == max(bloads)
    # no key split: the dQ pass reuses the forward section, every item maps to O
    assert (h.dq_tiles_offset, h.dq_slots_offset, h.n_dq_tiles) == (h.tiles_offset, h.slots_offset, h.n_tiles)
    assert h.n_merges == 0 and h.ws_rows == 0 and h.n_vitems == len(wl.items)
    assert not built.outmap()["to_workspace"].any() and not built.outmap()["o_shift"].any()


def _tile_array(tiles):
    return np.array([(t.q_row0, t.kv_row0, t.q_rows, t.kv_len, t.head, t.item) for t in tiles],
                    dtype=zl.TILE_DTYPE)


@pytest.mark.parametrize("cfg,kv_chunk,n_slots", [(0, 64, 0), (0, 64, 3), (0, 100, 7), (2, 8192, 256),
                                                  (3, 27456, 256), (3, 40000, 97), (3, 1 << 20, 256),
                                                  (3, -1, 256), (5, -1, 256), (6, -1, 97)])
def test_key_split_worklist_matches_reference(cfg, kv_chunk, n_slots):
    wl = W.config(cfg)
    built = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim,
                              n_slots=n_slots, kv_chunk=kv_chunk)
    h = built.header
    assert h.kv_chunk == kv_chunk
    ref, begin, loads = lpt_schedule(wl.items, h.block_m, n_slots, h.cost_c0, kv_chunk)
    assert h.n_tiles == len(ref) and np.array_equal(built.tiles(), _tile_array(ref))
    if n_slots:
        assert list(built.slots()) == begin and h.max_slot_cost == max(loads)
    outmap, merges, ws = split_plan(wl.items, kv_chunk)
    om = built.outmap()
    assert h.n_vitems == len(outmap)
    assert [(int(a), int(b)) for a, b in zip(om["o_shift"], om["to_workspace"])] == outmap
    got_m = built.merges()
    assert h.n_merges == len(merges)
    assert [tuple(int(x) for x in m) for m in got_m.tolist()] == merges
    assert h.ws_rows == ws
    assert built.workspace_floats == ws * wl.num_heads * (wl.head_dim + 1)
    # the dQ pass runs the unsplit forward schedule
    uref, ubegin, _ = lpt_schedule(wl.items, h.block_m, n_slots, h.cost_c0)
    assert h.n_dq_tiles == len(uref) and np.array_equal(built.dq_tiles(), _tile_array(uref))
    if n_slots:
        assert list(built.dq_slots()) == ubegin
    if merges:
        assert h.dq_tiles_offset not in (h.tiles_offset,)


def test_worklist_is_deterministic():
    wl = W.config(2)
    a = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, 24, 128, n_slots=256)
    b = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, 24, 128, n_slots=256)
    assert np.array_equal(a.host, b.host)


def _rc_build(items, q_rows=1000, kv_rows=1000, H=4, d=128, n_slots=0, scale=0.0, kv_chunk=0,
              buf=True, nbytes=None):
    arr, n = zl._items_array(items)
    prob = zl.Problem(q_rows, kv_rows, H, d, scale, kv_chunk)
    size = ctypes.c_size_t(0)
    rc = zl.lib.zl_build_worklist(ctypes.byref(prob), arr, n, n_slots, None, ctypes.byref(size))
    if rc or not buf:
        return rc
    host = np.zeros(size.value // 8 + 1, np.uint64)
    size2 = ctypes.c_size_t(size.value if nbytes is None else nbytes)
    return zl.lib.zl_build_worklist(ctypes.byref(prob), arr, n, n_slots, host.ctypes.data, ctypes.byref(size2))


def test_build_errors():
    ok = [(0, 10, 0, 10, 0, 4)]
    assert _rc_build(ok) == 0
    assert _rc_build(ok, d=96) == -2
    assert _rc_build(ok, H=0) == -2
    assert _rc_build([(995, 10, 0, 10, 0, 4)]) == -3           # rows past q_rows
    assert _rc_build([(0, 10, 995, 10, 0, 4)]) == -3           # keys past kv_rows
    assert _rc_build([(0, 10, 0, 10, 2, 3)]) == -3             # heads past H
    assert _rc_build([(0, -1, 0, 10, 0, 4)]) == -3
    assert _rc_build([(0, 10, 0, 10, 0, 2), (5, 10, 0, 10, 1, 2)]) == -4   # shared (row, head)
    assert _rc_build([(0, 10, 0, 10, 0, 2), (5, 10, 0, 10, 2, 2)]) == 0    # disjoint heads
    assert _rc_build([(0, 10, 0, 10, 0, 4), (10, 10, 0, 10, 0, 4)]) == 0   # adjacent rows
    assert _rc_build(ok, n_slots=-1) == -9
    assert _rc_build(ok, kv_chunk=-2) == -9
    assert _rc_build(ok, kv_chunk=-1) == 0  # ZL_KV_CHUNK_AUTO
    assert _rc_build(ok, kv_chunk=1) == 0
    assert _rc_build(ok, nbytes=64) == -5
    assert _rc_build(ok, scale=float("inf")) == -9
    prob = zl.Problem(10, 10, 1, 64, 0.0, 0)
    size = ctypes.c_size_t(0)
    assert zl.lib.zl_build_worklist(None, None, 0, 0, None, ctypes.byref(size)) == -1
    assert zl.lib.zl_build_worklist(ctypes.byref(prob), None, 1, 0, None, ctypes.byref(size)) == -1
    assert zl.lib.zl_build_worklist(ctypes.byref(prob), None, 0, 0, None, ctypes.byref(size)) == 0
    assert b"overlap" in zl.lib.zl_status_string(-4)


def test_empty_and_zero_length_items():
    wl = zl.build_worklist([(0, 0, 0, 5, 0, 2), (0, 3, 0, 0, 0, 2), (3, 4, 0, 5, 1, 0)], 10, 10, 2, 64)
    t = wl.tiles()
    assert wl.n_tiles == 2 and set(t["kv_len"]) == {0} and set(t["q_rows"]) == {3}


def test_fwd_and_merge_reject_bad_arguments_before_any_hip_call():
    wl = W.config(0)
    built = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim)
    p = 1 << 20  # aligned fake device address; never dereferenced on these paths
    f = zl.lib.zl_coalesced_attn_fwd
    assert f(None, p, p, p, p, p, p, None, None) == -1
    assert f(built.host_ptr(), None, p, p, p, p, p, None, None) == -1
    assert f(built.host_ptr(), p, p + 8, p, p, p, p, None, None) == -6
    bad = built.host.copy()
    bad[:4] = 0
    assert f(bad.ctypes.data, p, p, p, p, p, p, None, None) == -7
    bad = built.host.copy()
    bad.view(np.uint32)[1] = 99  # abi version
    assert f(bad.ctypes.data, p, p, p, p, p, p, None, None) == -7
    bad = built.host.copy()
    zl.WorklistHeader.from_buffer(bad).total_bytes = 64
    assert f(bad.ctypes.data, p, p, p, p, p, p, None, None) == -7
    bad = built.host.copy()
    zl.WorklistHeader.from_buffer(bad).n_merges = 1  # merges without a workspace size
    assert f(bad.ctypes.data, p, p, p, p, p, p, None, None) == -7
    split = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim, kv_chunk=64)
    assert split.header.ws_rows > 0
    assert f(split.host_ptr(), p, p, p, p, p, p, None, None) == -1       # workspace required
    assert f(split.host_ptr(), p, p, p, p, p, p, p + 4, None) == -6      # and aligned
    m = zl.lib.zl_merge_partials
    assert m(2, 10, 4, 0, 4, 128, None, p, 10, p, p, None) == -1
    assert m(2, 10, 4, 0, 4, 96, p, p, 10, p, p, None) == -2
    assert m(2, 10, 4, 2, 3, 128, p, p, 10, p, p, None) == -3
    assert m(0, 10, 4, 0, 4, 128, p, p, 10, p, p, None) == -9
    assert m(65, 10, 4, 0, 4, 128, p, p, 10, p, p, None) == -9   # more than 64 parts
    assert m(2, 10, 4, 0, 4, 128, p, p, 5, p, p, None) == -9   # stride < rows
    assert m(2, 10, 4, 0, 4, 128, p + 4, p, 10, p, p, None) == -6
    q = 1 << 30
    assert m(2, 10, 4, 0, 4, 128, p, q, 10, p, q + (1 << 24), None) == -9   # output overlaps parts


def test_mfma_calibration_rejects_bad_arguments_before_any_hip_call():
    c = zl.lib.zl_calib_mfma
    out = ctypes.c_double(0.0)
    assert c(0, 1000, None, None) == -1
    assert c(2, 1000, ctypes.byref(out), None) == -9
    assert c(-1, 1000, ctypes.byref(out), None) == -9
    assert c(0, 0, ctypes.byref(out), None) == -9
    assert c(1, (1 << 24) + 1, ctypes.byref(out), None) == -9
    assert out.value == 0.0
    with pytest.raises(ValueError):
        zl.calibrate_mfma("zeros")


def test_nan_and_oversized_shapes_are_rejected_by_the_shipped_library():
    """The host half of the shipped libzl.so keeps IEEE NaN semantics (it is
    built without the kernels' finite-math flag): a NaN softmax scale is
    rejected when the worklist is built and when a tampered header reaches
    the forward or backward entry point, before any HIP call. Rows of more
    than 2^20 elements (num_heads * head_dim) are rejected too, so the
    kernels' 32-bit in-buffer offsets cannot wrap."""
    ok = [(0, 10, 0, 10, 0, 4)]
    assert _rc_build(ok, scale=float("nan")) == -9
    assert _rc_build(ok, scale=float("-nan")) == -9
    assert _rc_build(ok, H=(1 << 20) // 128) == 0
    assert _rc_build([(0, 10, 0, 10, 0, 4)], H=(1 << 20) // 128 + 1) == -2
    assert _rc_build([(0, 10, 0, 10, 0, 4)], H=(1 << 20) // 64 + 1, d=64) == -2
    wl = W.config(0)
    built = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim)
    p = 1 << 20  # aligned fake device address; never dereferenced on these paths
    fwd, bwd = zl.lib.zl_coalesced_attn_fwd, zl.lib.zl_coalesced_attn_bwd
    for field, value in (("softmax_scale", float("nan")), ("softmax_scale", -1.0),
                         ("softmax_scale", 0.0), ("num_heads", (1 << 20) // 64 + 1)):
        bad = built.host.copy()
        setattr(zl.WorklistHeader.from_buffer(bad), field, value)
        assert fwd(bad.ctypes.data, p, p, p, p, p, p, None, None) == -7, field
        assert bwd(bad.ctypes.data, p, p, p, p, p, p, p, p, p, p, p, None) == -7, field
        assert b"header" in zl.lib.zl_last_error()


def test_noalloc_forward_rejects_bad_arguments_before_any_hip_call():
    """The allocation-free forward checks the worklist, pointers and the size
    of its key-chunk partials against the library's scratch on the host."""
    p = 1 << 20  # aligned fake device address; never dereferenced on these paths
    f = zl.lib.zl_coalesced_attn_fwd_noalloc
    wl = W.config(0)
    built = zl.build_worklist(wl.items, wl.q_rows, wl.kv_rows, wl.num_heads, wl.head_dim)
    assert f(None, p, p, p, p, p, p, None) == -1
    assert f(built.host_ptr(), None, p, p, p, p, p, None) == -1
    assert f(built.host_ptr(), p, p + 8, p, p, p, p, None) == -6
    bad = built.host.copy()
    zl.WorklistHeader.from_buffer(bad).softmax_scale = float("nan")
    assert f(bad.ctypes.data, p, p, p, p, p, p, None) == -7
    big = zl.build_worklist([(0, 6000, 0, 8000, 0, 24)], 6000, 8000, 24, 128, kv_chunk=2000)
    assert 4 * big.workspace_floats > zl.NOALLOC_SCRATCH_BYTES
    assert f(big.host_ptr(), p, p, p, p, p, p, None) == -5
    assert b"allocation-free" in zl.lib.zl_last_error()
    text = open(HEADER).read()
    assert zl.NOALLOC_SCRATCH_BYTES == eval(re.search(r"#define ZL_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)",
                                                      text).expand(r"\1 << \2"))

"""The allocation-free forward (zl_coalesced_attn_fwd_noalloc) against the
workspace entry point (zl_coalesced_attn_fwd) through the C ABI: two calls
in a row on worklists that split items into key chunks, the second smaller
than the first, each compared bit for bit with the workspace entry point and
with the fp64 oracle under the parity gates."""

import math

import numpy as np
import pytest

from coalesced_attention_amd import workloads as W

from gpu_util import Stats, log, oracle_compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case_large():
    # an 1300-query item against 8000 keys, split into 4 key chunks of 2048
    # (partials: 4 x 1300 rows x 24 heads x 129 floats = 64.4 MB of the
    # 64 MiB scratch), next to a whole 1024-token image and a short item
    H, d = 24, 128
    items = [W.Item(0, 1300, 0, 8000, 0, H), W.Item(1300, 1024, 8000, 1024, 0, H),
             W.Item(2324, 77, 9024, 300, 3, 9)]
    g = torch.Generator().manual_seed(71)
    q = torch.randn((2401, H, d), generator=g).to(torch.bfloat16)
    k = torch.randn((9324, H, d), generator=g).to(torch.bfloat16)
    v = torch.randn((9324, H, d), generator=g).to(torch.bfloat16)
    return items, q, k, v, H, d, 2000


def _case_small():
    wl = W.config(0)  # 3 sequences + a k=2 split, 2 heads, d=64; 64-key chunks
    inp = W.make_inputs(wl)
    return list(wl.items), inp.q, inp.k, inp.v, wl.num_heads, wl.head_dim, 64


def test_noalloc_forward_matches_the_workspace_entry_point_on_two_calls():
    from coalesced_attention_amd import zl
    dev = torch.device("cuda:0")
    for name, case in (("large", _case_large), ("small", _case_small)):
        items, q, k, v, H, d, kv_chunk = case()
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        built = zl.build_worklist(items, q.shape[0], k.shape[0], H, d, n_slots=zl.default_slots(dev),
                                  device=dev, kv_chunk=kv_chunk)
        assert built.header.n_merges > 0
        assert 4 * built.workspace_floats <= zl.NOALLOC_SCRATCH_BYTES
        log(f"no-alloc {name}: {built.n_tiles} tiles, {built.header.n_merges} split item(s), "
            f"partials {4 * built.workspace_floats / 2**20:.1f} MiB")
        nan = float("nan")
        o_ref = torch.full((q.shape[0], H, d), nan, device=dev)
        l_ref = torch.full((q.shape[0], H), nan, device=dev)
        zl.coalesced_attn_fwd(built, qd, kd, vd, o_ref, l_ref)
        o = torch.full_like(o_ref, nan)
        lse = torch.full_like(l_ref, nan)
        zl.coalesced_attn_fwd_noalloc(built, qd, kd, vd, o, lse)
        torch.cuda.synchronize()
        # the same kernels in the same order: the same bits, uncovered rows untouched
        assert torch.equal(torch.isnan(o), torch.isnan(o_ref))
        assert torch.equal(torch.nan_to_num(o, nan=7.0), torch.nan_to_num(o_ref, nan=7.0))
        assert torch.equal(torch.nan_to_num(lse, nan=7.0), torch.nan_to_num(l_ref, nan=7.0))
        st = oracle_compare(Stats(), items, q.float().numpy(), k.float().numpy(), v.float().numpy(),
                            o.cpu().numpy(), lse.cpu().numpy(), 1 / math.sqrt(d), seed=5)
        st.assert_gates(f"no-alloc forward, {name} call")


def test_noalloc_forward_rejects_oversized_partials_before_any_launch():
    from coalesced_attention_amd import zl
    dev = torch.device("cuda:0")
    H, d = 24, 128
    # 6000 queries x 4 key chunks x 24 heads x 129 floats: 297 MB > 64 MiB
    items = [W.Item(0, 6000, 0, 8000, 0, H)]
    built = zl.build_worklist(items, 6000, 8000, H, d, n_slots=16, device=dev, kv_chunk=2000)
    assert 4 * built.workspace_floats > zl.NOALLOC_SCRATCH_BYTES
    sentinel = 3.5
    q = torch.zeros((6000, H, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((8000, H, d), dtype=torch.bfloat16, device=dev)
    o = torch.full((6000, H, d), sentinel, device=dev)
    lse = torch.full((6000, H), sentinel, device=dev)
    with pytest.raises(zl.ZlError) as e:
        zl.coalesced_attn_fwd_noalloc(built, q, k, k, o, lse)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert torch.all(o == sentinel) and torch.all(lse == sentinel)

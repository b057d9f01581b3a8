"""CPU offload of position-free blocks (MiniPIC §3, contribution 5): whole blocks move
between the device pools and a pinned host pool with pic_blocks_copy, bytes unchanged,
and come back under other physical ids with no position bookkeeping."""

import numpy as np
import pytest

import position_independent_kv_amd as pic
from tests.gpu_harness import DeviceWorkload, to_f64
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _bits(t):
    torch = _torch()
    t = t.cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy().view(np.int32)


def _i32(a, dev):
    return _torch().from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


@pytest.mark.parametrize("case", ["bf16", "f32"])
def test_round_trip_through_pinned_host_is_bit_exact(case):
    torch = _torch()
    kw = dict(builder="decode", seed=51, R=5, seg_len=64, n_seg=3, n_shared=1, n_spans=5)
    if case == "f32":
        kw["dtype"] = "f32"
    w = make_workload("offload_" + case, **kw)
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    nb = w.num_blocks
    rng = np.random.default_rng(3)
    src = rng.permutation(nb)[: nb // 2 + 3].astype(np.int32)
    host_nb = len(src) + 7
    host_ids = rng.permutation(host_nb)[: len(src)].astype(np.int32)
    hk = torch.full((host_nb,) + tuple(dw.k_pool.shape[1:]), float("nan"), dtype=dw.dtype,
                    pin_memory=True)
    hv = torch.full((host_nb,) + tuple(dw.v_pool.shape[1:]), float("nan"), dtype=dw.dtype,
                    pin_memory=True)
    ids_src = _i32(src, "cuda")
    ids_host = _i32(host_ids, "cuda")
    pic.pic_blocks_copy(dw.k_pool, dw.v_pool, ids_src, hk, hv, ids_host)      # swap out
    torch.cuda.synchronize()
    k0, v0 = _bits(dw.k_pool), _bits(dw.v_pool)
    assert np.array_equal(_bits(hk)[host_ids], k0[src])
    assert np.array_equal(_bits(hv)[host_ids], v0[src])
    back = rng.permutation(nb + 5)[: len(src)].astype(np.int32)
    dk = torch.full((nb + 5,) + tuple(dw.k_pool.shape[1:]), 0.0, dtype=dw.dtype, device="cuda")
    dv = torch.full((nb + 5,) + tuple(dw.v_pool.shape[1:]), 0.0, dtype=dw.dtype, device="cuda")
    pic.pic_blocks_copy(hk, hv, ids_host, dk, dv, _i32(back, "cuda"))           # swap in
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dk)[back], k0[src])
    assert np.array_equal(_bits(dv)[back], v0[src])
    untouched = np.setdiff1d(np.arange(nb + 5), back)
    assert not _bits(dk)[untouched].any() and not _bits(dv)[untouched].any()


def test_out_of_range_pairs_are_skipped():
    torch = _torch()
    a = torch.randn(4, 2, 16, 64, device="cuda").to(torch.bfloat16)
    b = torch.randn(4, 2, 64, 16, device="cuda").to(torch.bfloat16)
    ka, va = torch.zeros_like(a), torch.zeros_like(b)
    pic.pic_blocks_copy(a, b, _i32([0, 5, -1, 2], "cuda"), ka, va, _i32([3, 0, 1, 9], "cuda"))
    torch.cuda.synchronize()
    assert torch.equal(ka[3], a[0]) and torch.equal(va[3], b[0])
    assert not ka[:3].any() and not va[:3].any()


@pytest.mark.parametrize("name,decode", [("c1d", True), ("offload_mixed", False)])
def test_attention_after_offload_and_remap_is_bit_identical(name, decode):
    """Swap every block out to the host, clobber the device pools, swap them back in under
    a random new numbering and remap the block tables: the outputs do not change by a bit."""
    torch = _torch()
    if name == "c1d":
        w = make_workload(name)
    else:
        w = make_workload(name, builder="mixed", seed=43, n_chunks=3, chunk=96, n_dec=6,
                          per_dec=2)
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    ref = to_f64(dw.attention(decode=decode, out=torch.empty_like(dw.q)))
    nb = w.num_blocks
    hk = torch.empty(tuple(dw.k_pool.shape), dtype=dw.dtype, pin_memory=True)
    hv = torch.empty(tuple(dw.v_pool.shape), dtype=dw.dtype, pin_memory=True)
    ident = _i32(np.arange(nb), "cuda")
    pic.pic_blocks_copy(dw.k_pool, dw.v_pool, ident, hk, hv, ident)
    dw.k_pool.fill_(float("nan"))
    dw.v_pool.fill_(float("nan"))
    perm = np.random.default_rng(9).permutation(nb).astype(np.int32)   # old id -> new id
    pic.pic_blocks_copy(hk, hv, ident, dw.k_pool, dw.v_pool, _i32(perm, "cuda"))
    bt = w.block_table.copy()
    dw.block_table = _i32(perm[bt], "cuda")
    got = to_f64(dw.attention(decode=decode, out=torch.empty_like(dw.q)))
    torch.cuda.synchronize()
    assert np.array_equal(got, ref)

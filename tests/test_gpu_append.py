"""pic_attn_decode_append: the decode launch writes each request's new token itself.

Request r's new token (row r of new_k / new_v) is its key slot seq_lens[r] - 1.  The
last key chunk of the request stores it into the pools and uses it for that slot in the
same launch.  The result must be what pic_cache_write of those rows followed by
pic_attn_decode gives: the same output bits and the same pool bytes (slots nobody writes
keep their NaN fill in both).
"""

import numpy as np
import pytest

import position_independent_kv_amd as pic
from tests.gpu_harness import DeviceWorkload, i32
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _bits(t):
    torch = _torch()
    w = torch.int16 if t.element_size() == 2 else torch.int32
    return t.contiguous().view(w).cpu().numpy()


def _pair(w, lens=None):
    """Separate write + decode on one copy of the batch, append on another.  lens: seq_lens
    to use instead of the batch's (each new token then goes to slot lens[r] - 1)."""
    torch = _torch()
    a, b = DeviceWorkload(w), DeviceWorkload(w)
    if lens is None:
        lens = np.asarray(w.seq_lens, np.int64)
        a.write_new_tokens()
    else:
        lens = np.asarray(lens, np.int64)
        for dw in (a, b):
            dw.seq_lens = i32(lens.astype(np.int32))
        bt = np.asarray(w.block_table, np.int64)
        slots = bt[np.arange(w.num_reqs), (lens - 1) // w.block_size] * w.block_size \
            + (lens - 1) % w.block_size
        pic.pic_cache_write(a.new_k, a.new_v, i32(slots.astype(np.int32)), a.k_pool, a.v_pool)
    out_a = a.attention(decode=True)
    pic.pic_attn_decode_append(b.q, b.new_k, b.new_v, b.q_pos, b.k_pool, b.v_pool,
                               b.block_table, b.seq_lens, b.cu_k, b.k_pos, b.cos, b.sin,
                               w.max_seq_len, b.out, b.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out_a), _bits(b.out)), "outputs differ"
    assert np.array_equal(_bits(a.k_pool), _bits(b.k_pool)), "K pools differ"
    assert np.array_equal(_bits(a.v_pool), _bits(b.v_pool)), "V pools differ"
    return out_a


CASES = {
    # 10 requests x (3 x 400-key segments, one a shared span) + the new token
    "bf16-d128-g4": dict(builder="decode", seed=71, R=10, seg_len=400, n_seg=3, n_shared=1,
                         n_spans=5),
    "bf16-d64-g8": dict(builder="decode", seed=72, R=6, seg_len=256, n_seg=3, n_shared=1,
                        n_spans=3, hq=64, hkv=8, d=64),
    "f32-d128-g2": dict(builder="decode", seed=73, R=5, seg_len=160, n_seg=3, n_shared=1,
                        n_spans=5, hq=8, hkv=4, dtype="f32"),
    "bf16-g1": dict(builder="decode", seed=74, R=4, seg_len=512, n_seg=2, n_shared=0, n_spans=0,
                    hq=8, hkv=8),
    # 6 kv heads: the second head group's workgroup has two idle waves
    "bf16-hkv6": dict(builder="decode", seed=77, R=5, seg_len=320, n_seg=2, n_shared=1,
                      n_spans=5, hq=24, hkv=6),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_equals_write_then_decode(name):
    w = make_workload("x", **CASES[name])
    out = _pair(w)
    assert np.isfinite(out.float().cpu().numpy()).all()


def test_append_at_every_kind_of_slot():
    """Private contexts cut to lengths whose new token is the first or last slot of a block,
    the only key, or the first or last key of a chunk (512-key chunks): 1, 2, 15, 16, 17,
    31-33, 511-513, 1023-1025, 1537 and 2049 keys."""
    w = make_workload("x", builder="decode", seed=75, R=16, seg_len=512, n_seg=4, n_shared=0,
                      n_spans=0)
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1023, 1024, 1025, 1537, 2049]
    assert max(lens) <= int(w.seq_lens.min())
    _pair(w, lens)


def test_append_full_size_decode_batch():
    """The 64 x 4097-key decode batch of the benchmark (tail blocks private)."""
    _pair(make_workload("c2"))


def test_append_decode_steps_in_a_row():
    """Three decode steps in a row, each appending one more token: every step's output and
    the final pools equal those of write + decode steps."""
    torch = _torch()
    w = make_workload("x", builder="decode", seed=76, R=6, seg_len=240, n_seg=2, n_shared=0,
                      n_spans=0)
    a, b = DeviceWorkload(w), DeviceWorkload(w)
    L0 = np.asarray(w.seq_lens, np.int64) - 2  # steps at L0, L0 + 1, L0 + 2 keys
    bt = np.asarray(w.block_table, np.int64)
    g = torch.Generator(device="cuda").manual_seed(5)
    for step in range(3):
        lens = L0 + step
        nk = torch.randn(a.new_k.shape, generator=g, device="cuda").to(a.new_k.dtype)
        nv = torch.randn(a.new_v.shape, generator=g, device="cuda").to(a.new_v.dtype)
        for dw in (a, b):
            dw.seq_lens = i32(lens.astype(np.int32))
        slots = bt[np.arange(w.num_reqs), (lens - 1) // w.block_size] * w.block_size \
            + (lens - 1) % w.block_size
        pic.pic_cache_write(nk, nv, i32(slots.astype(np.int32)), a.k_pool, a.v_pool)
        out_a = a.attention(decode=True)
        pic.pic_attn_decode_append(b.q, nk, nv, b.q_pos, b.k_pool, b.v_pool, b.block_table,
                                   b.seq_lens, b.cu_k, b.k_pos, b.cos, b.sin, w.max_seq_len,
                                   b.out, b.workspace)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_a), _bits(b.out)), step
    assert np.array_equal(_bits(a.k_pool), _bits(b.k_pool))
    assert np.array_equal(_bits(a.v_pool), _bits(b.v_pool))


def test_append_rejects_bad_rows():
    torch = _torch()
    w = make_workload("x", **CASES["bf16-g1"])
    b = DeviceWorkload(w)
    with pytest.raises(ValueError):
        pic.pic_attn_decode_append(b.q, b.new_k[:-1], b.new_v, b.q_pos, b.k_pool, b.v_pool,
                                   b.block_table, b.seq_lens, b.cu_k, b.k_pos, b.cos, b.sin,
                                   w.max_seq_len, b.out, b.workspace)
    with pytest.raises(TypeError):
        pic.pic_attn_decode_append(b.q, b.new_k.float(), b.new_v, b.q_pos, b.k_pool, b.v_pool,
                                   b.block_table, b.seq_lens, b.cu_k, b.k_pos, b.cos, b.sin,
                                   w.max_seq_len, b.out, b.workspace)
    torch.cuda.synchronize()

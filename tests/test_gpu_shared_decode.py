"""pic_attn_decode_shared: decode with block-determined key chunks, identical chunks of
different requests run side by side on one XCD.

Parity with the fp64 oracle (same tolerances as the other decode tests), bit-exact
indexing (needle), and the properties the chunking promises: a request's output does not
depend on the rest of the batch, and requests holding the same blocks give the same bits.
The blocks shared at different offsets are what MiniPIC §2.1 caches position-free.
"""

import numpy as np
import pytest

import position_independent_kv_amd as pic
from tests.gpu_harness import DeviceWorkload, i32, to_f64
from tests.oracle_harness import oracle_outputs, select_rows
from workloads import make_workload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}

SMALL = {
    "decode": dict(builder="decode", seed=61, R=9, seg_len=96, n_seg=4, n_shared=2, n_spans=6),
    "decode_long": dict(builder="decode", seed=62, R=3, seg_len=1120, n_seg=2, n_shared=1,
                        n_spans=3),
    "decode_g8_d64": dict(builder="decode", seed=63, R=5, seg_len=64, n_seg=3, n_shared=1,
                          n_spans=5, hq=16, hkv=2, d=64),
    "decode_g1": dict(builder="decode", seed=64, R=4, seg_len=32, n_seg=2, n_shared=0,
                      n_spans=0, hq=4, hkv=4),
    "decode_f32_d128": dict(builder="decode", seed=65, R=4, seg_len=544, n_seg=2, n_shared=1,
                            n_spans=4, dtype="f32"),
    "long_shared": dict(builder="long", seed=66, R=3, n_spans=12, span_len=512),
}


def _torch():
    import torch
    return torch


def _shared(w, dw=None):
    torch = _torch()
    dw = dw or DeviceWorkload(w)
    dw.write_new_tokens()
    out = torch.empty_like(dw.out)
    dw.attention_shared(out=out)
    torch.cuda.synchronize()
    return out, dw


def _bits(t):
    torch = _torch()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_parity(case):
    w = make_workload(case, **dict(SMALL[case]))
    out, dw = _shared(w)
    got = to_f64(out)
    err = float(np.abs(got - oracle_outputs(w)).max())
    # and close to the uniform-chunk decode (rounding only)
    base = to_f64(dw.attention())
    print(f"{case}: max abs err {err:.3e}; vs pic_attn_decode {np.abs(got - base).max():.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL[w.dtype]
    assert float(np.abs(got - base).max()) <= TOL[w.dtype]


@pytest.mark.parametrize("name,requests", [("c2", [0, 17, 63]), ("c4", [1])])
def test_full_size_sampled(name, requests):
    w = make_workload(name)
    out, _ = _shared(w)
    got = to_f64(out)
    ref = oracle_outputs(w, requests=requests)
    err = float(np.abs(select_rows(got, w, requests) - ref).max())
    print(f"{name}: max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL[w.dtype]


def test_request_alone_equals_request_in_batch():
    """The chunking depends only on the request's own block table."""
    torch = _torch()
    w = make_workload("x", **dict(SMALL["decode_long"]))
    out, dw = _shared(w)
    for r in range(w.num_reqs):
        L = int(w.seq_lens[r])
        one = torch.empty((1, w.hq, w.d), dtype=dw.dtype, device="cuda")
        ws = torch.zeros(pic.pic_attn_decode_shared_workspace_size(1, L, w.hq, w.hkv, w.d,
                                                                   dw.dtype),
                         dtype=torch.uint8, device="cuda")
        k0 = int(w.cu_seqlens_k[r])
        pic.pic_attn_decode_shared(dw.q[r:r + 1].contiguous(), dw.q_pos[r:r + 1].contiguous(),
                                   dw.k_pool, dw.v_pool, dw.block_table[r:r + 1].contiguous(),
                                   dw.seq_lens[r:r + 1].contiguous(), i32(np.array([0, L])),
                                   dw.k_pos[k0:k0 + L].contiguous(), dw.cos, dw.sin, L, one, ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(one[0]), _bits(out[r])), r


def test_identical_requests_give_identical_bits():
    """Several requests with the same block table, positions and query: the planner groups
    their chunks (same first block) and every copy must come out bit-identical."""
    torch = _torch()
    w = make_workload("x", **dict(SMALL["long_shared"]))
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    R = 6
    L = int(w.seq_lens[0])
    bt = dw.block_table[:1].expand(R, -1).contiguous()
    q = dw.q[:1].expand(R, -1, -1).contiguous()
    q_pos = dw.q_pos[:1].expand(R).contiguous()
    k_pos = dw.k_pos[:L].repeat(R).contiguous()
    seq = i32(np.full(R, L, np.int32))
    cu = i32((np.arange(R + 1) * L).astype(np.int32))
    out = torch.empty((R, w.hq, w.d), dtype=dw.dtype, device="cuda")
    ws = torch.zeros(pic.pic_attn_decode_shared_workspace_size(R, L, w.hq, w.hkv, w.d, dw.dtype),
                     dtype=torch.uint8, device="cuda")
    for _ in range(2):  # and the workspace may be reused as is
        pic.pic_attn_decode_shared(q, q_pos, dw.k_pool, dw.v_pool, bt, seq, cu, k_pos, dw.cos,
                                   dw.sin, L, out, ws)
        torch.cuda.synchronize()
        for r in range(1, R):
            assert torch.equal(_bits(out[r]), _bits(out[0])), r
    ref = oracle_outputs(w, requests=[0])
    assert float(np.abs(to_f64(out[:1]) - ref[:1]).max()) <= TOL[w.dtype]


@pytest.mark.parametrize("L", [1500, (1 << 20)])
def test_needle_every_region(L):
    """One non-zero key per request at slot j; the query shares its position, so the
    output is V[j] bit for bit, wherever the block-determined chunk boundaries fall.  The
    second case is the largest context the planner takes (65536 blocks)."""
    torch = _torch()
    rng = np.random.default_rng(17)
    hkv, G, d, B = 2, 4, 128, 16
    hq = hkv * G
    if L < 4096:
        slots = sorted(set(list(range(0, 40)) + [127, 128, 129, 383, 384, 575, 576, 577, 1023,
                                                 1024, 1311, 1498, 1499]))
    else:
        slots = [0, 4095, L // 2 + 3, L - 1]
    R = len(slots)
    nb_req = -(-L // B)
    nblocks = R * nb_req
    perm = rng.permutation(nblocks).astype(np.int32)
    block_table = perm.reshape(R, nb_req)
    k_pool = torch.zeros((nblocks, hkv, B, d), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.randn((nblocks, hkv, d, B), device="cuda").to(torch.bfloat16)
    max_pos = 9001
    t_pos = 5000
    k_pos = rng.integers(0, max_pos, size=(R, L)).astype(np.int32)
    qv = torch.randn((hkv, d))
    q1 = qv[:, None, :].expand(hkv, G, d).reshape(hq, d)
    qf = q1.to(torch.bfloat16).float().view(hkv, G, d)[:, 0, :]
    c = 200.0 * np.sqrt(d) / float((qf * qf).sum(-1).min())
    for r, j in enumerate(slots):
        k_pos[r, j] = t_pos
        k_pool[int(block_table[r, j // B]), :, j % B, :] = (qf * c).to(torch.bfloat16).cuda()
    cos = torch.empty((max_pos, d // 2), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    pic.pic_rope_table(cos, sin, 500000.0)
    q = q1[None].expand(R, hq, d).contiguous().to(torch.bfloat16).cuda()
    out = torch.empty_like(q)
    ws = torch.zeros(pic.pic_attn_decode_shared_workspace_size(R, L, hq, hkv, d, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    seq = np.full(R, L, np.int32)
    cu = (np.arange(R + 1, dtype=np.int64) * L).astype(np.int32)
    pic.pic_attn_decode_shared(q, i32(np.full(R, t_pos, np.int32)), k_pool, v_pool,
                               i32(block_table), i32(seq), i32(cu), i32(k_pos.reshape(-1)), cos,
                               sin, L, out, ws)
    torch.cuda.synchronize()
    for r, j in enumerate(slots):
        want = v_pool[int(block_table[r, j // B]), :, :, j % B]
        got = out[r].view(hkv, G, d)
        for h in range(hq):
            assert torch.equal(_bits(got[h // G, h % G]), _bits(want[h // G])), (r, j, h)

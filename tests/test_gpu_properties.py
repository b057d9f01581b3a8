"""GPU properties that must hold bit for bit (indexing, sharing, batching).

Each check compares two runs of the HIP library (through the C ABI) whose
results must be identical bytes, or compares against stored values chosen so
the floating-point result is exact (the needle).  The sharing checks follow
MiniPIC §2.1: one physical block serves several requests at different
offsets, never mutated by attention.
"""

import numpy as np
import pytest

import position_independent_kv_amd as pic
from tests.gpu_harness import DeviceWorkload, i32, to_torch
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _bits(t):
    torch = _torch()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same_bits(a, b):
    torch = _torch()
    return torch.equal(_bits(a), _bits(b))


SMALL_DEC = dict(builder="decode", seed=51, R=10, seg_len=400, n_seg=3, n_shared=1, n_spans=5)
SMALL_PRE = dict(builder="prefill", seed=52, R=3, n_spans=4, span_len=160, per_req=2, q_len=90)
SMALL_MIX = dict(builder="mixed", seed=53, n_chunks=3, chunk=128, n_dec=9, per_dec=2)


def _fresh(kw, name="x"):
    w = make_workload(name, **dict(kw))
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    return w, dw


# ---------------------------------------------------------------------------
# needle: a single huge score makes the output exactly that slot's V row
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 4), ("f32", 64, 1), ("bf16", 64, 8)])
def test_needle_every_slot_decode(dtype, d, G):
    """Request r puts one non-zero key at slot j_r; all other keys are zero.
    Query and needle key share one logical position, so the rotation cancels
    in the score (rotations preserve dot products) and the score is
    |q|^2 * c / sqrt(d) ~ 200: every other weight underflows to 0 and the
    output must equal V[j_r] bit for bit.  j_r sweeps every offset inside a
    block, block boundaries, chunk boundaries and the last slot."""
    torch = _torch()
    rng = np.random.default_rng(7)
    hkv = 2
    hq = hkv * G
    B = 16
    L = 1500                                     # several decode chunks
    dt = pic.PIC_F32 if dtype == "f32" else pic.PIC_BF16
    starts = [pic.pic_decode_chunk_start(L, k, dt) for k in range(1, pic.pic_decode_num_splits(L, dt))]
    edges = [x + e for x in starts for e in (-1, 0, 1)]  # chunk boundaries
    slots = sorted(set(list(range(0, 48)) + edges + [383, 384, 385, 575, 576, 767, 768, 1023,
                                                     1024, 1100, 1311, 1312, 1498, 1499]))
    R = len(slots)
    nb_req = -(-L // B)
    nblocks = R * nb_req + 3
    perm = rng.permutation(nblocks)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k_pool = torch.zeros((nblocks, hkv, B, d), dtype=tdt, device="cuda")
    v_pool = torch.randn((nblocks, hkv, d, B), dtype=torch.float32, device="cuda").to(tdt)
    block_table = np.zeros((R, nb_req), np.int32)
    for r in range(R):
        block_table[r] = perm[r * nb_req:(r + 1) * nb_req]
    t_pos = 5000
    k_pos = rng.integers(0, 9000, size=(R, L)).astype(np.int32)
    qv = torch.randn((R, hkv, d), dtype=torch.float32)
    q = qv[:, :, None, :].expand(R, hkv, G, d).reshape(R, hq, d).contiguous()
    q = q.to(tdt)
    qf = q.float().view(R, hkv, G, d)[:, :, 0, :]
    for r, j in enumerate(slots):
        k_pos[r, j] = t_pos
        c = 200.0 * np.sqrt(d) / float((qf[r] * qf[r]).sum(-1).min())
        blk, off = int(block_table[r, j // B]), j % B
        k_pool[blk, :, off, :] = (qf[r] * c).to(tdt).cuda()
    cos = torch.empty((9001, d // 2), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    pic.pic_rope_table(cos, sin, 500000.0)
    seq = np.full(R, L, np.int32)
    cu_k = np.concatenate([[0], np.cumsum(seq)]).astype(np.int32)
    out = torch.empty((R, hq, d), dtype=tdt, device="cuda")
    ws = torch.zeros(pic.pic_attn_workspace_size(R, R, L, hq, hkv, d, tdt), dtype=torch.uint8,
                     device="cuda")
    pic.pic_attn_decode(q.cuda(), i32(np.full(R, t_pos)), k_pool, v_pool, i32(block_table),
                        i32(seq), i32(cu_k), i32(k_pos.reshape(-1)), cos, sin, L, out, ws)
    torch.cuda.synchronize()
    for r, j in enumerate(slots):
        blk, off = int(block_table[r, j // B]), j % B
        for h in range(hq):
            want = v_pool[blk, h // G, :, off]
            assert _same_bits(out[r, h], want), (r, j, h)


@pytest.mark.parametrize("L,needles", [
    (200, [0, 17, 130, 131, 150, 199]),
    # 24 tiles over 4200 keys: each tile's keys are split into 4 chunks and merged
    (4200, [0, 1100, 2100, 4130, 4131, 4199]),
], ids=["short", "split-tiles"])
def test_needle_prefill_rows(L, needles):
    """Prefill: rows that can see the needle slot return V[j] exactly (also when the
    tile's keys are split into chunks: the other chunks' weights underflow to zero)."""
    torch = _torch()
    rng = np.random.default_rng(8)
    hkv, G, d, B = 2, 4, 128, 16
    hq = hkv * G
    ql = 70
    R = len(needles)
    nb_req = -(-L // B)
    nblocks = R * nb_req
    perm = rng.permutation(nblocks)
    k_pool = torch.zeros((nblocks, hkv, B, d), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.randn((nblocks, hkv, d, B), device="cuda").to(torch.bfloat16)
    block_table = perm.reshape(R, nb_req).astype(np.int32)
    t_pos = 777
    k_pos = rng.integers(0, 1000, size=(R, L)).astype(np.int32)
    qv = torch.randn((hkv, d))
    q1 = qv[:, None, :].expand(hkv, G, d).reshape(hq, d)
    q = q1[None].expand(R * ql, hq, d).contiguous().to(torch.bfloat16)
    qf = q[0].float().view(hkv, G, d)[:, 0, :]
    c = 200.0 * np.sqrt(d) / float((qf * qf).sum(-1).min())
    for r, j in enumerate(needles):
        k_pos[r, j] = t_pos
        k_pool[int(block_table[r, j // B]), :, j % B, :] = (qf * c).to(torch.bfloat16).cuda()
    q_pos = np.full(R * ql, t_pos, np.int32)
    cos = torch.empty((1001, d // 2), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    pic.pic_rope_table(cos, sin, 500000.0)
    seq = np.full(R, L, np.int32)
    cu_k = np.concatenate([[0], np.cumsum(seq)]).astype(np.int32)
    cu_q = (np.arange(R + 1) * ql).astype(np.int32)
    out = torch.empty_like(q.cuda())
    ws = torch.zeros(pic.pic_attn_workspace_size(R, R * ql, L, hq, hkv, d, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    pic.pic_attn_prefill(q.cuda(), i32(cu_q), i32(q_pos), k_pool, v_pool, i32(block_table),
                         i32(seq), i32(cu_k), i32(k_pos.reshape(-1)), cos, sin, ql, L, out, ws)
    torch.cuda.synchronize()
    checked = 0
    for r, j in enumerate(needles):
        blk, off = int(block_table[r, j // B]), j % B
        for i in range(ql):
            if j <= L - ql + i:     # the row sees the needle
                for h in range(hq):
                    assert _same_bits(out[r * ql + i, h], v_pool[blk, h // G, :, off]), (r, j, i, h)
                checked += 1
    assert checked > 0


# ---------------------------------------------------------------------------
# sharing and layout invariance (bit-exact)
# ---------------------------------------------------------------------------

def _rerun(dw, decode=None):
    torch = _torch()
    out = torch.empty_like(dw.out)
    dw.attention(decode=decode, out=out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kw", [SMALL_DEC, SMALL_PRE, SMALL_MIX], ids=["decode", "prefill", "mixed"])
def test_shared_blocks_equal_private_copies(kw):
    """Giving every request private copies of the blocks it references (no
    sharing at all) changes no output bit."""
    torch = _torch()
    w, dw = _fresh(kw)
    base = _rerun(dw)
    nb = -(-w.seq_lens.astype(np.int64) // w.block_size)
    stride = int(nb.max())
    new_bt = np.zeros((w.num_reqs, stride), np.int32)
    src = []
    for r in range(w.num_reqs):
        for i in range(int(nb[r])):
            new_bt[r, i] = len(src)
            src.append(int(w.block_table[r, i]))
    idx = torch.tensor(src, dtype=torch.long, device="cuda")
    dw.k_pool = dw.k_pool.index_select(0, idx).contiguous()
    dw.v_pool = dw.v_pool.index_select(0, idx).contiguous()
    dw.block_table = i32(new_bt)
    got = _rerun(dw)
    assert _same_bits(got, base)


@pytest.mark.parametrize("kw", [SMALL_DEC, SMALL_MIX], ids=["decode", "mixed"])
def test_physical_block_permutation_invariance(kw):
    torch = _torch()
    w, dw = _fresh(kw)
    base = _rerun(dw)
    perm = np.random.default_rng(3).permutation(w.num_blocks)
    inv = np.argsort(perm)
    # new_pool[perm[b]] = pool[b]
    dw.k_pool = dw.k_pool.index_select(0, torch.tensor(inv, device="cuda")).contiguous()
    dw.v_pool = dw.v_pool.index_select(0, torch.tensor(inv, device="cuda")).contiguous()
    dw.block_table = i32(perm[w.block_table])
    got = _rerun(dw)
    assert _same_bits(got, base)


@pytest.mark.parametrize("kw", [SMALL_DEC, SMALL_MIX], ids=["decode", "mixed"])
def test_attention_never_writes_the_pools(kw):
    torch = _torch()
    w, dw = _fresh(kw)
    k0, v0 = dw.k_pool.clone(), dw.v_pool.clone()
    _rerun(dw)
    _rerun(dw)
    assert _same_bits(dw.k_pool, k0) and _same_bits(dw.v_pool, v0)


def test_request_alone_equals_request_in_batch():
    """A request's decode output does not depend on the rest of the batch."""
    torch = _torch()
    w, dw = _fresh(SMALL_DEC)
    base = _rerun(dw)
    for r in [0, 4, w.num_reqs - 1]:
        L = int(w.seq_lens[r])
        one = torch.empty((1, w.hq, w.d), dtype=dw.dtype, device="cuda")
        ws = torch.zeros(pic.pic_attn_workspace_size(1, 1, L, w.hq, w.hkv, w.d, dw.dtype),
                         dtype=torch.uint8, device="cuda")
        k0 = int(w.cu_seqlens_k[r])
        pic.pic_attn_decode(dw.q[r:r + 1].contiguous(), dw.q_pos[r:r + 1].contiguous(),
                            dw.k_pool, dw.v_pool, dw.block_table[r:r + 1].contiguous(),
                            dw.seq_lens[r:r + 1].contiguous(), i32(np.array([0, L])),
                            dw.k_pos[k0:k0 + L].contiguous(), dw.cos, dw.sin, L, one, ws)
        torch.cuda.synchronize()
        assert _same_bits(one[0], base[r]), r


def test_decode_launch_equals_mixed_launch():
    """The same decode batch through pic_attn_decode and pic_attn_prefill."""
    w, dw = _fresh(SMALL_DEC)
    a = _rerun(dw, decode=True)
    b = _rerun(dw, decode=False)
    assert _same_bits(a, b)


def test_two_chunk_decode_items_equal_one_chunk_items():
    """A decode batch big enough for two-chunk work items (64 requests x 4097 keys: 1024
    single-chunk items, an even number per compute unit, so the decode launch walks two
    consecutive chunks per workgroup) equals, bit for bit, the same batch through the mixed
    launch, whose decode items take one chunk each, and a request decoded alone (one chunk
    per item): each chunk's partial is the same either way."""
    torch = _torch()
    w, dw = _fresh(dict(builder="decode", seed=29, R=64, seg_len=1024, n_seg=4, n_shared=2,
                        n_spans=32))
    a = _rerun(dw, decode=True)
    b = _rerun(dw, decode=False)
    assert torch.isfinite(a.float()).all()
    assert _same_bits(a, b)
    r = 5
    L = int(w.seq_lens[r])
    one = torch.empty((1, w.hq, w.d), dtype=dw.dtype, device="cuda")
    ws = torch.zeros(pic.pic_attn_workspace_size(1, 1, L, w.hq, w.hkv, w.d, dw.dtype),
                     dtype=torch.uint8, device="cuda")
    k0 = int(w.cu_seqlens_k[r])
    pic.pic_attn_decode(dw.q[r:r + 1].contiguous(), dw.q_pos[r:r + 1].contiguous(),
                        dw.k_pool, dw.v_pool, dw.block_table[r:r + 1].contiguous(),
                        dw.seq_lens[r:r + 1].contiguous(), i32(np.array([0, L])),
                        dw.k_pos[k0:k0 + L].contiguous(), dw.cos, dw.sin, L, one, ws)
    torch.cuda.synchronize()
    assert _same_bits(one[0], a[r])


def test_prefill_request_alone_equals_in_mixed_batch():
    torch = _torch()
    w, dw = _fresh(SMALL_MIX)
    base = _rerun(dw)
    ql = w.q_lens()
    r = int(np.nonzero(ql > 1)[0][0])
    q0, q1 = int(w.cu_seqlens_q[r]), int(w.cu_seqlens_q[r + 1])
    L = int(w.seq_lens[r])
    k0 = int(w.cu_seqlens_k[r])
    one = torch.empty((q1 - q0, w.hq, w.d), dtype=dw.dtype, device="cuda")
    ws = torch.zeros(pic.pic_attn_workspace_size(1, q1 - q0, L, w.hq, w.hkv, w.d, dw.dtype),
                     dtype=torch.uint8, device="cuda")
    pic.pic_attn_prefill(dw.q[q0:q1].contiguous(), i32(np.array([0, q1 - q0])),
                         dw.q_pos[q0:q1].contiguous(), dw.k_pool, dw.v_pool,
                         dw.block_table[r:r + 1].contiguous(), dw.seq_lens[r:r + 1].contiguous(),
                         i32(np.array([0, L])), dw.k_pos[k0:k0 + L].contiguous(), dw.cos, dw.sin,
                         q1 - q0, L, one, ws)
    torch.cuda.synchronize()
    assert _same_bits(one, base[q0:q1])


def test_workspace_reuse_across_calls_and_shapes():
    torch = _torch()
    w, dw = _fresh(SMALL_DEC)
    a = _rerun(dw)
    w2, dw2 = _fresh(SMALL_MIX)
    # the mixed batch borrows the first workspace if it is large enough
    need = pic.pic_attn_workspace_size(w2.num_reqs, w2.total_q, w2.max_seq_len, w2.hq, w2.hkv,
                                       w2.d, dw2.dtype)
    if dw.workspace.numel() >= need:
        dw2.workspace = dw.workspace
    _rerun(dw2)
    b = _rerun(dw)
    c = _rerun(dw)
    assert _same_bits(a, b) and _same_bits(b, c)


# ---------------------------------------------------------------------------
# degenerate shapes
# ---------------------------------------------------------------------------

def test_empty_batch_and_empty_context():
    torch = _torch()
    w, dw = _fresh(SMALL_DEC)
    # zero requests: no-op, no error
    pic.pic_attn_decode(dw.q[:0], dw.q_pos[:0], dw.k_pool, dw.v_pool, dw.block_table[:0],
                        dw.seq_lens[:0], dw.cu_k[:1], dw.k_pos, dw.cos, dw.sin, w.max_seq_len,
                        dw.out[:0], dw.workspace)
    # a request with seq_len 0 gets a zero row; its neighbours are unaffected
    base = _rerun(dw)
    sl = w.seq_lens.copy()
    sl[2] = 0
    cu = np.concatenate([[0], np.cumsum(sl)]).astype(np.int32)
    kp = np.concatenate([w.k_pos[w.cu_seqlens_k[r]:w.cu_seqlens_k[r] + sl[r]]
                         for r in range(w.num_reqs)]).astype(np.int32)
    dw.seq_lens, dw.cu_k, dw.k_pos = i32(sl), i32(cu), i32(kp)
    got = _rerun(dw)
    assert torch.count_nonzero(got[2].float()) == 0
    keep = [r for r in range(w.num_reqs) if r != 2]
    assert _same_bits(got[keep], base[keep])


def test_single_key_context():
    """seq_len 1: the output is that key's V row exactly (softmax of one score)."""
    torch = _torch()
    w, dw = _fresh(SMALL_DEC)
    sl = np.ones(w.num_reqs, np.int32)
    cu = np.arange(w.num_reqs + 1, dtype=np.int32)
    kp = np.array([w.k_pos[w.cu_seqlens_k[r]] for r in range(w.num_reqs)], np.int32)
    dw.seq_lens, dw.cu_k, dw.k_pos = i32(sl), i32(cu), i32(kp)
    got = _rerun(dw)
    G = w.hq // w.hkv
    for r in range(w.num_reqs):
        blk = int(w.block_table[r, 0])
        for h in range(w.hq):
            assert _same_bits(got[r, h], dw.v_pool[blk, h // G, :, 0]), (r, h)


@pytest.mark.parametrize("events", ["torch", "timing"])
@pytest.mark.parametrize("kw", [SMALL_DEC, SMALL_MIX], ids=["decode", "mixed"])
def test_kernel_events_bracket_the_main_kernel(kw, events):
    """With the measurement hook set, the call's results are unchanged and the events
    span the main kernel only: a positive time no longer than the whole call.  Both kinds
    of event: torch's and the library's timing events."""
    torch = _torch()
    w, dw = _fresh(kw)
    base = _rerun(dw)
    if events == "torch":
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    else:
        ev = [pic.TimingEvent() for _ in range(4)]
    stream = torch.cuda.current_stream()
    pic.pic_set_kernel_events(ev[2], ev[3])
    try:
        ev[0].record(stream)
        out = torch.empty_like(dw.out)
        dw.attention(out=out)
        ev[1].record(stream)
    finally:
        pic.pic_set_kernel_events(None, None)
    torch.cuda.synchronize()
    assert _same_bits(out, base)
    kern, call = ev[2].elapsed_time(ev[3]), ev[0].elapsed_time(ev[1])
    assert 0.0 < kern <= call
    # with the hook off the events are left alone
    before = ev[2].elapsed_time(ev[3])
    _rerun(dw)
    assert ev[2].elapsed_time(ev[3]) == before


@pytest.mark.parametrize("kind", ["decode", "prefill", "mixed"])
def test_needle_at_maximum_sizes(kind):
    """Indexing at sizes far past the benchmark configs: 3 requests of 2^20 + 37 keys each
    (65,539 blocks per request, 196,617 in the pool, ~3.2 GB of K/V), positions drawn from
    [0, 2^21) with a 2^21 + 1-row table (1 GiB).  One needle per request, at the first slot,
    in the middle and at the last slot; the query shares the needle's position, so its
    score dominates and every row that sees it must return that slot's V row bit for bit.
    Prefill runs 40 query rows per request: 6 tiles, so each tile's keys are split into
    chunks merged by the combine launch.  Mixed runs requests 0 and 2 as one-row decodes
    (2,731 key chunks each: more than the planner's 1024 chunk-count groups, so its decode
    items are listed in request order) beside request 1's 40 rows in one prefill launch."""
    torch = _torch()
    rng = np.random.default_rng(11)
    hkv, G, d, B = 2, 4, 128, 16
    hq = hkv * G
    L = (1 << 20) + 37
    max_pos = (1 << 21) + 1
    needles = [0, L // 2 + 5, L - 1]
    R = len(needles)
    nb_req = -(-L // B)
    nblocks = R * nb_req
    perm = rng.permutation(nblocks).astype(np.int32)
    block_table = perm.reshape(R, nb_req)
    k_pool = torch.zeros((nblocks, hkv, B, d), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.randn((nblocks, hkv, d, B), device="cuda").to(torch.bfloat16)
    t_pos = max_pos - 1
    k_pos = rng.integers(0, max_pos - 1, size=(R, L)).astype(np.int32)
    qv = torch.randn((hkv, d))
    q1 = qv[:, None, :].expand(hkv, G, d).reshape(hq, d)
    qf = q1.to(torch.bfloat16).float().view(hkv, G, d)[:, 0, :]
    c = 200.0 * np.sqrt(d) / float((qf * qf).sum(-1).min())
    for r, j in enumerate(needles):
        k_pos[r, j] = t_pos
        k_pool[int(block_table[r, j // B]), :, j % B, :] = (qf * c).to(torch.bfloat16).cuda()
    cos = torch.empty((max_pos, d // 2), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    pic.pic_rope_table(cos, sin, 500000.0)
    seq = np.full(R, L, np.int32)
    cu_k = (np.arange(R + 1, dtype=np.int64) * L).astype(np.int32)
    qls = {"decode": [1] * R, "prefill": [40] * R, "mixed": [1, 40, 1]}[kind]
    cu_q_h = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    total_q = int(cu_q_h[-1])
    q = q1[None].expand(total_q, hq, d).contiguous().to(torch.bfloat16).cuda()
    q_pos = i32(np.full(total_q, t_pos, np.int32))
    out = torch.full_like(q, float("nan"))
    ws = torch.zeros(pic.pic_attn_workspace_size(R, total_q, L, hq, hkv, d, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    args = (k_pool, v_pool, i32(block_table), i32(seq), i32(cu_k), i32(k_pos.reshape(-1)),
            cos, sin)
    if kind == "decode":
        pic.pic_attn_decode(q, q_pos, *args, L, out, ws)
    else:
        pic.pic_attn_prefill(q, i32(cu_q_h), q_pos, *args, max(qls), L, out, ws)
    torch.cuda.synchronize()
    if kind == "mixed":
        assert pic.pic_decode_num_splits(L) >= 1024
    checked = 0
    for r, j in enumerate(needles):
        want = v_pool[int(block_table[r, j // B]), :, :, j % B]
        ql = qls[r]
        for i in range(ql):
            if j <= L - ql + i:  # the row sees the needle
                got = out[int(cu_q_h[r]) + i].view(hkv, G, d)
                for h in range(hq):
                    assert _same_bits(got[h // G, h % G], want[h // G]), (kind, r, j, i, h)
                checked += 1
    assert checked >= R


def test_mixed_launch_over_1024_requests():
    """A prefill launch of 1,104 requests (4 causal span prefills + 1,100 two-chunk decodes
    over those spans, in shuffled order): the planner handles requests in passes of 1024,
    so the later requests' items come from its second pass.  Every output row is compared
    with the oracle (outputs start as NaN, so a dropped item fails)."""
    from tests.gpu_harness import run_workload
    from tests.oracle_harness import oracle_outputs
    w = make_workload("x", builder="mixed", seed=61, n_chunks=4, chunk=208, n_dec=1100,
                      per_dec=4)
    assert w.num_reqs > 1024 and pic.pic_decode_num_splits(int(w.seq_lens.max())) == 2
    got = run_workload(w)
    assert np.isfinite(got).all()
    err = float(np.abs(got - oracle_outputs(w)).max())
    print(f"1104 requests: max abs err {err:.3e}")
    assert err <= 2e-2


def _tile_keys(L, ql, k, G, rows=256):
    """Keys tile k of a request sees: up to the causal limit of its last query row."""
    return min(L, L - ql + min((k * rows + rows - 1) // G, ql - 1) + 1)


@pytest.mark.parametrize("case", ["mixed", "c3", "split", "many"])
def test_work_list_holds_every_item_once_longest_first(case):
    """The mixed launch's work list, read back from the workspace (int[2] at byte 0, the
    item count first; int4 items from byte 256: kind | split << 4 | nsplit << 16, request,
    kv head (prefill) or head group (decode), tile or chunk).  Every prefill tile of every
    kv head and every decode chunk appears exactly once.  With 256 tiles or more (no key
    splitting) the list is longest first across both kinds: the tiles that see at least
    2,048 keys by 64-key bucket, then the decode chunks in one contiguous run, then the
    shorter tiles by bucket; the kv heads of one tile sit next to each other in head
    order.  A launch with fewer tiles splits each tile's keys into chunks (one item each)
    and keeps every prefill item ahead of the decode chunks (a split item's partial slot
    is its list position).  'mixed': 4 causal 4096-token span prefills (tiles of 64 to
    4,096 keys) and 24 decodes over two of those spans; 'c3': 8 chunked prefills of 512
    queries over 4,096 cached keys; 'split': one causal 2048-token span prefill with 2 kv
    heads (64 tiles, so 2 key chunks per tile) and 6 decodes over that span; 'many': 4
    causal 2048-token span prefills and 1,100 decodes cut to seeded lengths of 1 to 4,097
    keys (1 to 8 chunks), so the planner takes its requests in two passes of 1024 and
    every wave holds requests of both kinds.  The decode run, its interleave over the
    XCDs undone (dispatch position p holds logical item x * q + min(x, rem) + k for
    x = p % 8, k = p // 8, where q, rem = divmod(chunks, 8)), lists the requests with more
    chunks first, and inside one chunk count all requests' chunk 0, then chunk 1, ..."""
    torch = _torch()
    if case == "mixed":
        w = make_workload("x", values=False, builder="mixed", seed=63, n_chunks=4, chunk=4096,
                          n_dec=24, per_dec=2)
    elif case == "split":
        w = make_workload("x", values=False, builder="mixed", seed=64, n_chunks=1, chunk=2048,
                          n_dec=6, per_dec=1, hq=8, hkv=2)
    elif case == "many":
        w = make_workload("x", values=False, builder="mixed", seed=65, n_chunks=4, chunk=2048,
                          n_dec=1100, per_dec=2)
        dec = w.q_lens() == 1
        w.seq_lens[dec] = np.random.default_rng(65).integers(1, int(w.seq_lens.max()) + 1,
                                                             int(dec.sum()))
    else:
        w = make_workload(case, values=False)
    dw = DeviceWorkload(w, write_context=False)
    dw.k_pool.normal_()
    dw.v_pool.normal_()
    dw.attention(decode=False)
    torch.cuda.synchronize()
    ws = dw.workspace.cpu().numpy()
    n = int(ws[:4].view(np.int32)[0])
    items = ws[256:256 + 16 * n].view(np.int32).reshape(n, 4)
    G = w.hq // w.hkv
    ql, L = w.q_lens(), w.seq_lens
    tiles = sum(-(-int(q) * G // 256) for q in ql if q > 1) * w.hkv
    split = max(1, 256 // tiles) if tiles < 256 else 1     # chunks a long tile may take
    nsp = [max(1, min(split, int(L[r]) // 1024)) for r in range(w.num_reqs)]
    want_pf = {(r, g, k, sp) for r in range(w.num_reqs) if ql[r] > 1
               for k in range(-(-int(ql[r]) * G // 256)) for g in range(w.hkv)
               for sp in range(nsp[r])}
    want_dc = {(r, 0, c) for r in range(w.num_reqs) if ql[r] == 1
               for c in range(pic.pic_decode_num_splits(int(L[r])))}
    kind = items[:, 0] & 15
    sp_of, ns_of = (items[:, 0] >> 4) & 0xfff, (items[:, 0] >> 16) & 0xfff
    pf = [(int(it[1]), int(it[2]), int(it[3]), int(s))
          for it, s in zip(items[kind == 0], sp_of[kind == 0])]
    dc = [tuple(int(v) for v in it[1:]) for it in items[kind == 1]]
    assert len(pf) == len(set(pf)) and set(pf) == want_pf
    assert len(dc) == len(set(dc)) and set(dc) == want_dc
    for it, ns in zip(items[kind == 0], ns_of[kind == 0]):
        assert ns == (nsp[it[1]] if nsp[it[1]] > 1 else 0)
    if case == "split":
        assert max(nsp) > 1
        assert (kind[:len(pf)] == 0).all(), "a splitting launch keeps prefill items first"
        return
    assert tiles >= 256 and max(nsp) == 1
    # decode chunks: one contiguous run
    pos = np.flatnonzero(kind == 1)
    if len(pos):
        assert (np.diff(pos) == 1).all()
        d0, d1 = int(pos[0]), int(pos[-1]) + 1
    else:
        d0 = d1 = n
    buckets = np.array([min(_tile_keys(int(L[r]), int(ql[r]), k, G) >> 6, 1023)
                        if kd == 0 else -1 for kd, r, k in zip(kind, items[:, 1], items[:, 3])])
    before, after = buckets[:d0], buckets[d1:]
    assert (before >= 32).all() and (after < 32).all() and (after >= 0).all()
    for part in (before, after):
        assert (np.diff(part) <= 0).all(), "prefill tiles longest first"
    # the kv heads of a tile: adjacent, in head order (one item per tile and head here)
    for part0 in (0, d1):
        part = items[part0:d0 if part0 == 0 else n]
        assert len(part) % w.hkv == 0
        grp = part.reshape(-1, w.hkv, 4)
        assert (grp[:, :, 1] == grp[:, :1, 1]).all() and (grp[:, :, 3] == grp[:, :1, 3]).all()
        assert (grp[:, :, 2] == np.arange(w.hkv)[None, :]).all()
    # decode run in logical order: chunk count non-increasing; inside one count, chunk
    # index non-decreasing
    nd = d1 - d0
    q8, rem = divmod(nd, 8)
    p = np.arange(nd)
    logical = (p % 8) * q8 + np.minimum(p % 8, rem) + p // 8
    assert (np.sort(logical) == p).all()
    run = np.empty((nd, 2), np.int64)
    run[logical, 0] = [pic.pic_decode_num_splits(int(L[r])) for r in items[d0:d1, 1]]
    run[logical, 1] = items[d0:d1, 3]
    assert (np.diff(run[:, 0]) <= 0).all(), "requests with more chunks first"
    same = np.diff(run[:, 0]) == 0
    assert (np.diff(run[:, 1])[same] >= 0).all(), "chunk-major inside one chunk count"
    print(f"{case}: {len(pf)} prefill items ({len(before)} before the {len(dc)} decode "
          f"chunks in {len(set(run[:, 0].tolist()))} chunk counts, {len(after)} after)")


def test_refused_work_list_fills_nan():
    """Metadata that break a precondition (cu_seqlens_q descending between requests, so
    the rows of requests 0, 2, 4, ... overlap) make the work list larger than the
    workspace was sized for.  The planner then runs nothing and the launch fills every
    output row with NaN instead of leaving stale values; the call itself returns PIC_OK
    (the violation is device data).  With PIC_VALIDATE=1 the binding refuses the call."""
    import os
    torch = _torch()
    w, dw = _fresh(dict(builder="prefill", seed=62, R=9, n_spans=4, span_len=512, per_req=2,
                        q_len=512))
    T = 512
    cu_q = np.array([0] + [T if r % 2 == 0 else 0 for r in range(9)], np.int32)
    q = dw.q[:T].contiguous()
    out = torch.zeros_like(q)
    ws = torch.zeros(pic.pic_attn_workspace_size(9, T, w.max_seq_len, w.hq, w.hkv, w.d,
                                                 torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    args = (q, i32(cu_q), dw.q_pos[:T].contiguous(), dw.k_pool, dw.v_pool, dw.block_table,
            dw.seq_lens, dw.cu_k, dw.k_pos, dw.cos, dw.sin, T, w.max_seq_len, out, ws)
    pic.pic_attn_prefill(*args)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    os.environ["PIC_VALIDATE"] = "1"
    try:
        with pytest.raises(ValueError, match="q_len"):
            pic.pic_attn_prefill(*args)
    finally:
        del os.environ["PIC_VALIDATE"]
    # the same workspace then serves a valid call: request 0's 512 rows alone, which equal
    # its rows of the whole batch bit for bit
    cu_ok = np.array([0] + [T] * 9, np.int32)
    pic.pic_attn_prefill(q, i32(cu_ok), *args[2:])
    full = dw.attention()
    torch.cuda.synchronize()
    assert _same_bits(out, full[:T])


@pytest.mark.parametrize("kw", [SMALL_DEC, SMALL_PRE, SMALL_MIX], ids=["decode", "prefill", "mixed"])
def test_validate_mode_accepts_valid_batches(kw, monkeypatch):
    """PIC_VALIDATE=1 runs the host checks before every launch: valid batches pass them and
    give the same bytes as without the checks."""
    torch = _torch()
    w, dw = _fresh(kw)
    ref = dw.attention(out=torch.full_like(dw.q, float("nan")))
    monkeypatch.setenv("PIC_VALIDATE", "1")
    got = dw.attention(out=torch.full_like(dw.q, float("nan")))
    rot = dw.build_rotated_cache().attention_rotated(out=torch.full_like(dw.q, float("nan")))
    torch.cuda.synchronize()
    assert _same_bits(got, ref)
    assert torch.isfinite(rot.float()).all()


def test_stream_read_helper_orders():
    """The streaming-read measurement helper over a buffer front to back, as a permutation
    of 16 KiB pieces, and with piece ids outside the buffer (read as its last piece): each
    call completes and stores nothing (the sink keeps its fill)."""
    torch = _torch()
    g = torch.Generator(device="cuda")
    g.manual_seed(5)  # fixed data: whether a lane's folded word hits the store constant is fixed
    x = torch.randint(0, 255, (64 << 20,), dtype=torch.uint8, device="cuda", generator=g)
    sink = torch.full((512 * 256,), 7, dtype=torch.int32, device="cuda")
    n = (64 << 20) // 16384
    perm = torch.from_numpy(np.random.default_rng(1).permutation(n).astype(np.int32)).cuda()
    bad = perm.clone()
    bad[::3] = n + 5
    bad[1::3] = -2
    pic.pic_stream_read(x, 512, sink)
    pic.pic_stream_read(x, 512, sink, perm, 16384)
    pic.pic_stream_read(x, 512, sink, bad, 16384)
    torch.cuda.synchronize()
    assert bool((sink == 7).all())

"""Concurrent requests over shared blocks (MiniPIC §2.1: one physical block serves
concurrent requests at different offsets; §3: the design avoids races on a shared
cache because attention never writes the blocks).

Two streams of default priority, each with its own workspace, run attention over
request batches that read the same physical blocks at different logical offsets, many
calls interleaved so their kernels overlap on the device.  Every output must equal
the same batch run alone, bit for bit, and the pools must keep their bytes.
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
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


class SubBatch:
    """Requests `reqs` of a resident workload as a batch of their own (same pools)."""

    def __init__(self, dw, reqs):
        torch = _torch()
        w = dw.w
        self.dw = dw
        reqs = np.asarray(reqs)
        cu_q = w.cu_seqlens_q
        ql = (cu_q[reqs + 1] - cu_q[reqs]).astype(np.int64)
        rows = np.concatenate([np.arange(cu_q[r], cu_q[r + 1]) for r in reqs])
        L = w.seq_lens[reqs].astype(np.int64)
        kp = np.concatenate([w.k_pos[w.cu_seqlens_k[r]:w.cu_seqlens_k[r] + w.seq_lens[r]]
                             for r in reqs])
        self.decode = bool((ql == 1).all())
        self.q = dw.q[torch.from_numpy(rows).cuda()].contiguous()
        self.q_pos = i32(w.q_pos[rows])
        self.cu_q = i32(np.concatenate([[0], np.cumsum(ql)]))
        self.bt = i32(w.block_table[reqs])
        self.seq_lens = i32(L)
        self.cu_k = i32(np.concatenate([[0], np.cumsum(L)]))
        self.k_pos = i32(kp)
        self.max_q_len = int(ql.max())
        self.max_seq_len = int(L.max())
        tdt = dw.dtype
        n = pic.pic_attn_workspace_size(len(reqs), rows.shape[0], self.max_seq_len, w.hq, w.hkv,
                                        w.d, tdt)
        self.ws = torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda")

    def run(self, out, stream=None):
        dw = self.dw
        if self.decode:
            pic.pic_attn_decode(self.q, self.q_pos, dw.k_pool, dw.v_pool, self.bt, self.seq_lens,
                                self.cu_k, self.k_pos, dw.cos, dw.sin, self.max_seq_len, out,
                                self.ws, stream=stream)
        else:
            pic.pic_attn_prefill(self.q, self.cu_q, self.q_pos, dw.k_pool, dw.v_pool, self.bt,
                                 self.seq_lens, self.cu_k, self.k_pos, dw.cos, dw.sin,
                                 self.max_q_len, self.max_seq_len, out, self.ws, stream=stream)
        return out


def _concurrent_equals_serial(dw, batch_a, batch_b, reps=12):
    torch = _torch()
    pools = (dw.k_pool.clone(), dw.v_pool.clone())
    serial = [b.run(torch.full_like(b.q, float("nan"))) for b in (batch_a, batch_b)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    outs = [[torch.full_like(b.q, float("nan")) for _ in range(reps)]
            for b in (batch_a, batch_b)]
    cur = torch.cuda.current_stream()
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    for k in range(reps):                                # interleaved, so kernels overlap
        batch_a.run(outs[0][k], stream=s1)
        batch_b.run(outs[1][k], stream=s2)
    torch.cuda.synchronize()
    for i, b in enumerate((batch_a, batch_b)):
        for k in range(reps):
            assert torch.equal(_bits(outs[i][k]), _bits(serial[i])), (i, k)
    assert torch.equal(_bits(dw.k_pool), _bits(pools[0]))
    assert torch.equal(_bits(dw.v_pool), _bits(pools[1]))


def test_two_streams_decode_batches_sharing_spans():
    """c2's shape at 16 requests: every shared span is held by requests in both batches,
    each at its own offset."""
    w = make_workload("x", builder="decode", seed=81, R=16, seg_len=1024, n_seg=4, n_shared=2,
                      n_spans=8)
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    # split so that every span has users in both batches
    spans_of = [set(map(int, w.block_table[r, ::64])) for r in range(w.num_reqs)]
    a = list(range(0, w.num_reqs, 2))
    b = list(range(1, w.num_reqs, 2))
    shared = set().union(*[spans_of[r] for r in a]) & set().union(*[spans_of[r] for r in b])
    assert shared, "the two batches must read common blocks"
    _concurrent_equals_serial(dw, SubBatch(dw, a), SubBatch(dw, b))


def test_two_streams_span_prefill_beside_decodes():
    """A mixed prefill launch (span prefills + some decodes) on one stream and a decode
    batch over the same span blocks on the other."""
    w = make_workload("x", builder="mixed", seed=82, n_chunks=4, chunk=1024, n_dec=24,
                      per_dec=3)
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    ql = w.q_lens()
    pre = [int(r) for r in np.nonzero(ql > 1)[0]]
    dec = [int(r) for r in np.nonzero(ql == 1)[0]]
    _concurrent_equals_serial(dw, SubBatch(dw, pre + dec[:8]), SubBatch(dw, dec[8:]))

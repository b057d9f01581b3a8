"""pic_attn_decode_noalloc: the decode call whose chunk partials live in the library's
fixed per-device scratch array instead of a caller workspace (for callers that cannot
allocate).  Same kernels as pic_attn_decode, so the outputs must agree bit for bit."""

import numpy as np
import pytest

import position_independent_kv_amd as pic
from tests.gpu_harness import DeviceWorkload
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _bits(t):
    return t.view(_torch().int16) if t.dtype == _torch().bfloat16 else t.view(_torch().int32)


def _noalloc(dw, out):
    w = dw.w
    pic.pic_attn_decode_noalloc(dw.q, dw.q_pos, dw.k_pool, dw.v_pool, dw.block_table,
                                dw.seq_lens, dw.cu_k, dw.k_pos, dw.cos, dw.sin, w.max_seq_len,
                                out)
    return out


@pytest.mark.parametrize("first,second", [
    # multi-chunk bf16 requests, then a smaller batch with a different head layout
    (dict(builder="decode", seed=71, R=12, seg_len=800, n_seg=3, n_shared=1, n_spans=4),
     dict(builder="decode", seed=72, R=3, seg_len=160, n_seg=2, n_shared=0, n_spans=0,
          hq=16, hkv=2, d=64)),
    # fp32, then a smaller bf16 batch
    (dict(builder="decode", seed=73, R=6, seg_len=544, n_seg=2, n_shared=1, n_spans=3,
          dtype="f32"),
     dict(builder="decode", seed=74, R=2, seg_len=96, n_seg=2, n_shared=0, n_spans=0)),
], ids=["bf16-then-smaller", "f32-then-smaller-bf16"])
def test_noalloc_equals_workspace_decode_on_two_calls(first, second):
    torch = _torch()
    for n, kw in enumerate([first, second]):
        w = make_workload(f"noalloc{n}", **dict(kw))
        dw = DeviceWorkload(w)
        dw.write_new_tokens()
        ref = dw.attention()                      # pic_attn_decode, caller workspace
        got = _noalloc(dw, torch.full_like(dw.q, float("nan")))
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(_bits(got), _bits(ref)), n
        del dw


def test_noalloc_full_size_decode_matches_and_refuses_oversized_batches():
    """The c2 decode batch (64 x 4097 keys) fits the scratch and matches bit for bit; a
    batch whose partials exceed the 64 MiB array is refused on the host (nothing runs, the
    output keeps its contents)."""
    torch = _torch()
    w = make_workload("c2")
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    ref = dw.attention()
    got = _noalloc(dw, torch.full_like(dw.q, float("nan")))
    torch.cuda.synchronize()
    assert torch.equal(_bits(got), _bits(ref))
    keep = torch.full_like(dw.q, 3.0)
    wide = torch.zeros((w.num_reqs, 1 << 16), dtype=torch.int32, device="cuda")
    wide[:, :dw.block_table.shape[1]] = dw.block_table   # room for 2^20 keys per request
    with pytest.raises(pic.PicError) as e:
        pic.pic_attn_decode_noalloc(dw.q, dw.q_pos, dw.k_pool, dw.v_pool, wide, dw.seq_lens,
                                    dw.cu_k, dw.k_pos, dw.cos, dw.sin, 1 << 20, keep)
    assert e.value.status == pic.PIC_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((keep == 3.0).all())


def test_noalloc_step_replays_from_a_hip_graph():
    """What the entry point is for: a decode step (cache write + attention) captured in a
    HIP graph with no workspace to allocate, replayed four times with eager work (the
    workspace decode, which writes different memory) between replays; every replay equals
    the eager result bit for bit.  The first call on a device looks up the array's address
    (hipGetSymbolAddress), so it is made before capturing."""
    torch = _torch()
    w = make_workload("noalloc_graph", builder="decode", seed=75, R=8, seg_len=400, n_seg=3,
                      n_shared=1, n_spans=4)
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    eager = _noalloc(dw, torch.full_like(dw.q, float("nan"))).clone()
    static_out = torch.empty_like(dw.q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the side stream, outside the graph
        dw.write_new_tokens()
        _noalloc(dw, static_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dw.write_new_tokens()
        _noalloc(dw, static_out)
    for i in range(4):
        static_out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(static_out), _bits(eager)), i
        other = dw.attention(out=torch.empty_like(dw.q))
        torch.cuda.synchronize()
        assert torch.equal(_bits(other), _bits(eager)), i

"""A serving step (cache write + attention) captured in a HIP graph and replayed.

The library allocates nothing, issues no memset and keeps every launch on the caller's
stream, so a step can be captured once and replayed; each replay must reproduce the eager
result bit for bit, with other work on the stream between replays.
"""

import pytest

from tests.gpu_harness import DeviceWorkload
from workloads import make_workload

pytestmark = pytest.mark.gpu

CASES = {
    "decode": dict(builder="decode", seed=71, R=8, seg_len=400, n_seg=3, n_shared=1, n_spans=4),
    "mixed": dict(builder="mixed", seed=72, n_chunks=3, chunk=160, n_dec=6, per_dec=2),
}


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("case", sorted(CASES))
def test_step_replays_from_a_hip_graph(case):
    import torch
    w = make_workload(case, **dict(CASES[case]))
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    eager = dw.attention().clone()
    static_out = torch.empty_like(dw.out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's side, outside the graph
        dw.write_new_tokens()
        dw.attention(out=static_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dw.write_new_tokens()
        dw.attention(out=static_out)
    other = torch.empty_like(dw.out)
    for i in range(4):
        static_out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(static_out), _bits(eager)), i
        dw.attention(out=other)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(_bits(other), _bits(eager)), i


def test_decode_step_with_append_replays_from_a_hip_graph():
    """A decode step as one pic_attn_decode_append call (the launch writes the new tokens),
    captured and replayed: every replay rewrites the same slots with the same rows and must
    give the eager output bit for bit, with eager steps between replays."""
    import torch
    w = make_workload("decode", **dict(CASES["decode"]))
    dw = DeviceWorkload(w)
    assert dw.appends_new_tokens()
    eager = dw.attention_append().clone()
    static_out = torch.empty_like(dw.out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dw.attention_append(out=static_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dw.attention_append(out=static_out)
    other = torch.empty_like(dw.out)
    for i in range(4):
        static_out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(static_out), _bits(eager)), i
        dw.attention_append(out=other)
        torch.cuda.synchronize()
        assert torch.equal(_bits(other), _bits(eager)), i

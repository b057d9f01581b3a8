"""Prefill tiles split along the keys.

A mixed launch with fewer prefill tiles than compute units splits each
long-context tile into key chunks that run as separate work items and are
merged afterwards.  These batches trigger it (few tiles, contexts of 2048
keys and more) and are checked against the fp64 oracle; the needle test in
test_gpu_properties checks the split path bit for bit.
"""

import numpy as np
import pytest

import position_independent_kv_amd as pic
from workloads import make_trace, make_workload

pytestmark = pytest.mark.gpu

TOL = 2e-2

CASES = {
    # 1 request, 64 suffix rows over 4096 context keys: 8 tiles, 4 chunks each
    "one-request": dict(builder="prefill", seed=31, R=1, n_spans=4, span_len=1024, per_req=4,
                        q_len=64),
    # 2 requests, 300 rows over 3072: 80 tiles, 3 chunks each (ragged last tile)
    "two-requests": dict(builder="prefill", seed=32, R=2, n_spans=6, span_len=1024, per_req=3,
                         q_len=300),
    # head size 64, group 8 (64 q heads over 8 kv heads): 8 x 4 tiles, 3 chunks
    "d64-g8": dict(builder="prefill", seed=33, R=1, n_spans=3, span_len=1024, per_req=3,
                   q_len=100, hq=64, hkv=8, d=64),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_split_prefill_matches_oracle(name):
    from tests.gpu_harness import run_workload
    from tests.oracle_harness import oracle_outputs
    w = make_workload(name, **dict(CASES[name]))
    print(f"case {name}: {w.num_reqs} requests, q_lens {w.q_lens().tolist()}, "
          f"seq_lens {w.seq_lens.tolist()}", flush=True)
    got = run_workload(w)
    ref = oracle_outputs(w)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    assert err <= TOL, err


def test_split_prompts_beside_decodes():
    """Scheduled steps mixing final-prompt chunks over long contexts with decodes: the
    launch both merges decode chunks and split prompt tiles; every token of the trace
    is checked against the oracle, under both policies."""
    import torch
    from tests.gpu_harness import TraceRun
    from tests.oracle_harness import trace_token_outputs
    trace = make_trace("long", data_seed=41, n_spans=5, n_req=4, span_blocks=(64, 96),
                       spans_per_req=(2, 3), prompt=(20, 70), output=(2, 4), arrival_every=3,
                       arrivals_per_wave=2)
    print(f"trace {trace.description}", flush=True)
    n_span_tok = int(sum(trace.span_lens))
    tokens = np.concatenate([np.arange(0, n_span_tok, 13), np.arange(n_span_tok, trace.n_tokens)])
    ref = None
    for policy in (pic.PIC_SCHED_ISPS, pic.PIC_SCHED_BARRIER):
        tr = TraceRun(trace, policy, 256, 4, 2048)
        tr.run()
        torch.cuda.synchronize()
        out, _ = tr.outputs()
        assert np.isfinite(out).all()
        if ref is None:
            ref = trace_token_outputs(trace, tokens)
        err = float(np.abs(out[tokens] - ref).max())
        assert err <= TOL, (policy, err)

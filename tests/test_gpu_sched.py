"""Scheduled traces through the HIP path: ISPS and the barrier policy give the same
outputs (bit for bit where a token goes through the same kernel path), and every
token's output matches the fp64 oracle."""

import numpy as np
import pytest

import position_independent_kv_amd as pic
from workloads import make_trace

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _run(trace, policy, budget, max_running, num_blocks):
    import torch
    from tests.gpu_harness import TraceRun
    tr = TraceRun(trace, policy, budget, max_running, num_blocks)
    tr.run()
    torch.cuda.synchronize()
    return tr.outputs()


@pytest.mark.parametrize("budget,max_running,num_blocks", [(64, 4, 256), (40, 2, 28)])
def test_policies_agree_and_match_oracle(budget, max_running, num_blocks):
    from tests.oracle_harness import trace_token_outputs
    trace = make_trace("small", data_seed=11, n_spans=6, n_req=8)
    print(f"trace {trace.description}; budget {budget}, running {max_running}, "
          f"blocks {num_blocks}", flush=True)
    out_i, single_i = _run(trace, pic.PIC_SCHED_ISPS, budget, max_running, num_blocks)
    out_b, single_b = _run(trace, pic.PIC_SCHED_BARRIER, budget, max_running, num_blocks)
    assert not np.isnan(out_i).any() and not np.isnan(out_b).any()
    same = single_i == single_b
    assert same.mean() > 0.9
    assert np.array_equal(out_i[same], out_b[same])
    assert np.abs(out_i - out_b).max() <= TOL
    ref = trace_token_outputs(trace, np.arange(trace.n_tokens))
    assert np.abs(out_i - ref).max() <= TOL
    assert np.abs(out_b - ref).max() <= TOL

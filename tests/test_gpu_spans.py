"""End to end over span-aware block tables (MiniPIC §2.2 primitives feeding §2.1's kernel).

Prompts are composed of a context, SSEP spans drawn from a shared pool (padded to
blocks), a PDEP suffix and a ragged tail.  pic_build_block_tables decides the
sharing; each physical block's K/V is written once (slot -1 skips the repeats);
the attention kernels then read shared blocks at each request's own offsets.
Checked against the fp64 oracle (2e-2, bf16) and, bit for bit, against the same
batch laid out with private copies of every block.
"""

import numpy as np
import pytest

import position_independent_kv_amd as pic
from tests.gpu_harness import run_workload
from tests.oracle_harness import oracle_outputs
from workloads import Workload
from workloads.synth import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

B = 16
SSEP, PDEP = 128001, 128002
HQ, HKV, D = 8, 2, 128


def _prompts(rng, n_reqs=6):
    spans = [[SSEP] + rng.integers(0, 120000, size=int(rng.integers(1, 4)) * B - 1).tolist()
             for _ in range(5)]
    out = []
    for _ in range(n_reqs):
        body = rng.integers(0, 120000, size=int(rng.integers(0, 3)) * B).tolist()
        for k in rng.choice(len(spans), size=3, replace=False):
            body += spans[int(k)]
        body += [PDEP] + rng.integers(0, 120000, size=B - 1).tolist()
        body += rng.integers(0, 120000, size=int(rng.integers(1, B))).tolist()
        out.append(body)
    return out


def _workload(seed, kind, private=False):
    rng = np.random.default_rng(seed)
    prompts = _prompts(rng)
    lens = np.asarray([len(p) for p in prompts], np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    toks = np.concatenate([np.asarray(p, np.int32) for p in prompts])
    if private:  # every request's blocks private: one table build per request
        res = {"block_table": [], "k_pos": [], "slot_mapping": []}
        first = 0
        for r, p in enumerate(prompts):
            one = pic.pic_build_block_tables(np.asarray(p, np.int32),
                                             np.asarray([0, len(p)], np.int32), B, -1, -1,
                                             seed=1000 + r, first_block=first)
            res["block_table"].append(one["block_table"][0])
            res["k_pos"].append(one["k_pos"])
            res["slot_mapping"].append(one["slot_mapping"])
            first += one["num_new_blocks"]
        stride = max(len(x) for x in res["block_table"])
        bt = np.zeros((len(prompts), stride), np.int32)
        for r, row in enumerate(res["block_table"]):
            bt[r, :len(row)] = row
        k_pos = np.concatenate(res["k_pos"])
        slots = np.concatenate(res["slot_mapping"])
        nblocks = first
    else:
        res = pic.pic_build_block_tables(toks, cu, B, SSEP, PDEP, seed=3)
        bt, k_pos, slots, nblocks = (res["block_table"], res["k_pos"], res["slot_mapping"],
                                     res["num_new_blocks"])
    # token values are drawn per physical slot of the shared layout, so a shared block
    # holds the same numbers for every request and the private layout copies them
    shared = pic.pic_build_block_tables(toks, cu, B, SSEP, PDEP, seed=3)
    nphys = shared["num_new_blocks"]
    kv_rng = np.random.default_rng(100 + seed)
    kp = kv_rng.standard_normal((nphys * B, HKV, D), dtype=np.float32)
    vp = kv_rng.standard_normal((nphys * B, HKV, D), dtype=np.float32)
    phys = np.concatenate([shared["block_table"][r, np.arange(lens[r]) // B] * B
                           + np.arange(lens[r]) % B for r in range(len(prompts))])
    ctx_k = f32_to_bf16_bits(kp[phys])
    ctx_v = f32_to_bf16_bits(vp[phys])
    if kind == "decode":
        q_lens = np.ones(len(prompts), np.int64)
        q_pos = lens.astype(np.int32)              # the next position after the prompt
    else:
        q_lens = np.minimum(lens, B + 5)            # the PDEP suffix block and the tail
        q_pos = np.concatenate([np.arange(lens[r] - q_lens[r], lens[r])
                                for r in range(len(prompts))]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = f32_to_bf16_bits(kv_rng.standard_normal((int(cu_q[-1]), HQ, D), dtype=np.float32))
    empty = np.zeros((0, HKV, D), np.uint16)
    return Workload(
        name=f"spans{seed}{'p' if private else ''}", kind=kind, dtype="bf16", hq=HQ, hkv=HKV,
        d=D, block_size=B, base=500000.0, num_blocks=int(nblocks), max_pos=int(lens.max()) + 2,
        ctx_k=ctx_k, ctx_v=ctx_v, ctx_slots=np.asarray(slots, np.int32), new_k=empty,
        new_v=empty, new_slots=np.zeros(0, np.int32), q=q, cu_seqlens_q=cu_q, q_pos=q_pos,
        block_table=np.asarray(bt, np.int32), seq_lens=lens.astype(np.int32), cu_seqlens_k=cu,
        k_pos=np.asarray(k_pos, np.int32), description="span composition")


@pytest.mark.parametrize("kind", ["decode", "prefill"])
@pytest.mark.parametrize("seed", [0, 1])
def test_span_tables_attention_matches_oracle(kind, seed):
    w = _workload(seed, kind)
    assert w.num_blocks < sum(-(-int(x) // B) for x in w.seq_lens)  # blocks really shared
    got = run_workload(w)
    ref = oracle_outputs(w)
    err = float(np.abs(got - ref).max())
    print(f"spans {kind} seed {seed}: {w.num_blocks} physical blocks, max abs err {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_span_tables_shared_equal_private(kind):
    shared = run_workload(_workload(0, kind))
    private = run_workload(_workload(0, kind, private=True))
    assert np.array_equal(shared, private)

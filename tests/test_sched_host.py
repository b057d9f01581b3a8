"""Interleaved span-prefill scheduling (pic_sched_*): host tests, no GPU.

The scheduler's output is checked by replaying every step on a model of the
cache: each query row's token is written to its slot, then every key slot of
every sequence in the step must hold exactly the token the composed sequence
has there (a span token for the spans' part, the request's own token after).
That pins block allocation, sharing, eviction, positions and the causal
ordering of spans -> final prompt -> decodes, for both policies.
"""

import numpy as np
import pytest

import position_independent_kv_amd as pic

SPAN, PROMPT, DECODE = pic.PIC_SEQ_SPAN, pic.PIC_SEQ_PROMPT, pic.PIC_SEQ_DECODE


def make(policy, spans, reqs, budget=64, max_running=8, num_blocks=256, stride=64,
         max_seqs=64, max_keys=1 << 16):
    s = pic.Scheduler(policy, budget, max_running, num_blocks, max_seqs=max_seqs,
                      max_keys=max_keys, block_table_stride=stride)
    for n in spans:
        s.add_span(n)
    for r in reqs:
        s.add_request(*r)
    return s


def run_all(s, limit=10000):
    steps = []
    while True:
        st = s.step()
        if st is None:
            return steps
        steps.append(st)
        assert len(steps) < limit


def replay(spans, reqs, steps, policy, budget, num_blocks):
    """Check every step against a model of the cache; returns per-request event steps."""
    cache = {}
    span_off = []
    for (_, sids, _, _) in reqs:
        offs, o = [], 0
        for sid in sids:
            offs.append(o)
            o += spans[sid]
        span_off.append((offs, o))
    prompt_rows = {r: [] for r in range(len(reqs))}
    decode_steps = {r: [] for r in range(len(reqs))}
    span_last = {}
    prompt_first = {}
    for st in steps:
        n = st["num_seqs"]
        assert st["total_q"] <= budget
        kinds = set(st["seq_kind"].tolist())
        if policy == pic.PIC_SCHED_BARRIER:
            assert len(kinds) <= 1
        if n == 0:
            continue
        status, msg = pic.pic_validate_metadata(
            st["cu_seqlens_q"], st["q_pos"], st["block_table"], st["seq_lens"],
            st["cu_seqlens_k"], st["k_pos"], max_seq_len=st["max_seq_len"], max_pos=1 << 20,
            num_blocks=num_blocks)
        assert status == pic.PIC_OK, msg
        # the step's writes
        written = set()
        for i in range(n):
            kind, sid, qb = int(st["seq_kind"][i]), int(st["seq_id"][i]), int(st["q_begin"][i])
            a, b = st["cu_seqlens_q"][i], st["cu_seqlens_q"][i + 1]
            for t in range(b - a):
                c = qb + t
                assert st["q_pos"][a + t] == c
                slot = int(st["slot_mapping"][a + t])
                assert slot not in written, "two tokens of one step share a slot"
                written.add(slot)
                cache[slot] = ("span", sid, c) if kind == SPAN else ("req", sid, c)
        # every key slot of every sequence holds the composed sequence's token
        for i in range(n):
            kind, sid, qb = int(st["seq_kind"][i]), int(st["seq_id"][i]), int(st["q_begin"][i])
            L = int(st["seq_lens"][i])
            ql = int(st["cu_seqlens_q"][i + 1] - st["cu_seqlens_q"][i])
            assert L == qb + ql
            kp = st["k_pos"][st["cu_seqlens_k"][i]:st["cu_seqlens_k"][i + 1]]
            assert np.array_equal(kp, np.arange(L))
            bt = st["block_table"][i]
            for j in range(L):
                got = cache.get(int(bt[j // 16]) * 16 + j % 16)
                if kind == SPAN:
                    want = ("span", sid, j)
                else:
                    offs, stok = span_off[sid]
                    if j < stok:
                        k = max(x for x in range(len(offs)) if offs[x] <= j)
                        want = ("span", reqs[sid][1][k], j - offs[k])
                    else:
                        want = ("req", sid, j)
                assert got == want, (st["step"], kind, sid, j, got, want)
            if kind == SPAN:
                span_last[sid] = st["step"]
            elif kind == PROMPT:
                prompt_first.setdefault(sid, st["step"])
                prompt_rows[sid].extend(range(qb, qb + ql))
                for s_ in reqs[sid][1]:
                    assert span_last.get(s_, -1) < st["step"], "prompt before its spans"
            else:
                assert ql == 1
                decode_steps[sid].append(st["step"])
    for r, (arr, sids, P, O) in enumerate(reqs):
        stok = span_off[r][1]
        assert prompt_rows[r] == list(range(stok, stok + P)), r
        assert len(decode_steps[r]) == O
        assert all(b > a for a, b in zip(decode_steps[r], decode_steps[r][1:]))
        if P and O:
            assert decode_steps[r][0] > prompt_first[r]
        first = prompt_first.get(r, decode_steps[r][0] if O else None)
        if first is not None:
            assert first >= arr
    return decode_steps


SPANS = [32, 48]
REQS = [(0, [0, 1], 20, 3), (0, [1], 5, 2), (2, [0], 0, 2)]


def summary(steps):
    return [[(int(k), int(i), int(q), int(L)) for k, i, q, L in
             zip(st["seq_kind"], st["seq_id"], st["q_begin"], st["seq_lens"])] for st in steps]


def test_isps_hand_worked_schedule():
    """Budget 64; span 0 (32 tokens) and span 1 (48); r0 = spans 0,1 + 20 prompt + 3 out,
    r1 = span 1 + 5 + 2, r2 (arrives at step 2) = span 0 + no prompt + 2 out.
    Step 0 fills the budget with span 0 and 32 tokens of span 1; step 1 the rest of span 1.
    At step 2 r2 is admitted with its span resident and decodes at once, beside both
    final prompts; then one decode per running request per step."""
    s = make(pic.PIC_SCHED_ISPS, SPANS, REQS)
    got = summary(run_all(s))
    assert got == [
        [(SPAN, 0, 0, 32), (SPAN, 1, 0, 32)],
        [(SPAN, 1, 32, 48)],
        [(DECODE, 2, 32, 33), (PROMPT, 0, 80, 100), (PROMPT, 1, 48, 53)],
        [(DECODE, 0, 100, 101), (DECODE, 1, 53, 54), (DECODE, 2, 33, 34)],
        [(DECODE, 0, 101, 102), (DECODE, 1, 54, 55)],
        [(DECODE, 0, 102, 103)],
    ]


def test_barrier_hand_worked_schedule():
    """Same trace, one kind per step: the final prompts get a step of their own and r2's
    decodes wait behind them."""
    s = make(pic.PIC_SCHED_BARRIER, SPANS, REQS)
    got = summary(run_all(s))
    assert got == [
        [(SPAN, 0, 0, 32), (SPAN, 1, 0, 32)],
        [(SPAN, 1, 32, 48)],
        [(PROMPT, 0, 80, 100), (PROMPT, 1, 48, 53)],
        [(DECODE, 0, 100, 101), (DECODE, 1, 53, 54), (DECODE, 2, 32, 33)],
        [(DECODE, 0, 101, 102), (DECODE, 1, 54, 55), (DECODE, 2, 33, 34)],
        [(DECODE, 0, 102, 103)],
    ]


def random_trace(rng, n_spans, n_req, max_arrival):
    spans = [16 * int(rng.integers(1, 9)) for _ in range(n_spans)]
    reqs = []
    for _ in range(n_req):
        k = int(rng.integers(0, 4))
        sids = [int(x) for x in rng.choice(n_spans, size=k, replace=False)] if k else []
        P = int(rng.integers(0 if k else 1, 40))
        reqs.append((int(rng.integers(0, max_arrival + 1)), sids, P, int(rng.integers(0, 6))))
    return spans, reqs


@pytest.mark.parametrize("policy", [pic.PIC_SCHED_ISPS, pic.PIC_SCHED_BARRIER])
@pytest.mark.parametrize("seed", range(6))
def test_random_traces_replay(policy, seed):
    rng = np.random.default_rng(seed)
    spans, reqs = random_trace(rng, 6, 14, 12)
    budget = int(rng.integers(8, 100))
    s = make(policy, spans, reqs, budget=budget, max_running=int(rng.integers(1, 8)))
    steps = run_all(s)
    replay(spans, reqs, steps, policy, budget, 256)
    assert sum(st["num_finished"] for st in steps) == len(reqs)


@pytest.mark.parametrize("policy", [pic.PIC_SCHED_ISPS, pic.PIC_SCHED_BARRIER])
def test_eviction_and_prefill_again(policy):
    """A pool of 10 blocks, one request at a time, spans of 4 blocks: r0 (spans 0, 1) leaves
    both resident; r1 (span 2) needs 5 blocks with 2 free, so the least recently used idle
    span (0) is evicted; r2 (span 0) evicts span 1 and prefills span 0 again; r3 (spans 1, 2)
    evicts span 0 and prefills span 1 again, reusing the resident span 2.  Every read still
    sees the right tokens."""
    spans = [64, 64, 64]
    reqs = [(0, [0, 1], 8, 2), (0, [2], 8, 2), (0, [0], 8, 2), (0, [1, 2], 8, 1)]
    s = make(policy, spans, reqs, budget=32, max_running=1, num_blocks=10)
    steps = run_all(s)
    replay(spans, reqs, steps, policy, 32, 10)
    prefills = {}
    for st in steps:
        for k, i, a, b in zip(st["seq_kind"], st["seq_id"], st["cu_seqlens_q"][:-1],
                              st["cu_seqlens_q"][1:]):
            if k == SPAN:
                prefills[int(i)] = prefills.get(int(i), 0) + int(b - a)
    assert prefills == {0: 128, 1: 128, 2: 64}


def test_shared_span_is_prefilled_once():
    spans = [128]
    reqs = [(0, [0], 16, 1) for _ in range(6)]
    for policy in (pic.PIC_SCHED_ISPS, pic.PIC_SCHED_BARRIER):
        steps = run_all(make(policy, spans, reqs, budget=48))
        n = sum(int(b - a) for st in steps for k, a, b in
                zip(st["seq_kind"], st["cu_seqlens_q"][:-1], st["cu_seqlens_q"][1:]) if k == SPAN)
        assert n == 128


def test_isps_overlaps_decodes_with_new_spans():
    """A request arriving while others decode: ISPS keeps the decodes going in the same
    steps as the new span's prefill; the barrier policy stalls them."""
    spans = [256, 256]
    reqs = [(0, [0], 16, 12), (4, [1], 16, 4)]
    res = {}
    for policy in (pic.PIC_SCHED_ISPS, pic.PIC_SCHED_BARRIER):
        steps = run_all(make(policy, spans, reqs, budget=64))
        replay(spans, reqs, steps, policy, 64, 256)
        mixed = sum(1 for st in steps if len(set(st["seq_kind"].tolist())) > 1)
        res[policy] = (len(steps), mixed)
    assert res[pic.PIC_SCHED_ISPS][1] > 0 and res[pic.PIC_SCHED_BARRIER][1] == 0
    assert res[pic.PIC_SCHED_ISPS][0] < res[pic.PIC_SCHED_BARRIER][0]


def test_idle_steps_until_arrival():
    steps = run_all(make(pic.PIC_SCHED_ISPS, [16], [(3, [0], 4, 1)]))
    assert [st["num_seqs"] for st in steps[:3]] == [0, 0, 0]
    assert steps[3]["seq_kind"].tolist() == [SPAN]
    assert [st["step"] for st in steps] == list(range(len(steps)))


def test_argument_errors():
    with pytest.raises(pic.PicError):
        pic.pic_sched_create(7, 64, 4, 64)
    with pytest.raises(pic.PicError):
        pic.pic_sched_create(pic.PIC_SCHED_ISPS, 64, 4, 64, block_size=32)
    for bad in [(pic.PIC_SCHED_ISPS, 64, 4, 0), (pic.PIC_SCHED_ISPS, 0, 4, 64), (pic.PIC_SCHED_ISPS, 64, 0, 64)]:
        with pytest.raises(pic.PicError):
            pic.pic_sched_create(*bad)
    s = pic.Scheduler(pic.PIC_SCHED_ISPS, 64, 4, 8, max_seqs=8, max_keys=1024,
                      block_table_stride=8)
    with pytest.raises(pic.PicError):
        s.add_span(20)                      # not whole blocks
    sid = s.add_span(32)
    with pytest.raises(pic.PicError):
        s.add_request(0, [sid + 1], 4, 1)   # unknown span
    with pytest.raises(pic.PicError):
        s.add_request(0, [], 0, 3)          # nothing to attend to
    with pytest.raises(pic.PicError):
        s.add_request(0, [sid], 200, 0)     # more blocks than the pool
    with pytest.raises(pic.PicError):
        s.add_request(-1, [sid], 4, 1)
    s.add_request(0, [sid], 4, 1)
    assert s.step() is not None
    with pytest.raises(pic.PicError):
        s.add_span(16)                      # after stepping started


def test_too_small_arrays_leave_the_state_unchanged():
    spans, reqs = [64, 32], [(0, [0, 1], 24, 3), (1, [1], 8, 2)]
    ref = summary(run_all(make(pic.PIC_SCHED_ISPS, spans, reqs)))
    s = make(pic.PIC_SCHED_ISPS, spans, reqs)
    got = []
    for _ in range(len(ref)):
        for caps in [(1, 64, 8, 2), (64, 64, 16, 64), (64, 64, 1 << 16, 1)]:
            with pytest.raises(pic.PicError):
                pic.pic_sched_step(s.handle, *caps)
        got.append(s.step())
    assert s.step() is None
    assert summary(got) == ref


@pytest.mark.parametrize("budget,max_running,num_blocks", [(64, 4, 256), (40, 2, 28)])
@pytest.mark.parametrize("policy", [pic.PIC_SCHED_ISPS, pic.PIC_SCHED_BARRIER])
def test_gpu_test_traces_replay(policy, budget, max_running, num_blocks):
    """The schedules the GPU tests execute: valid metadata, right tokens in every slot, and
    every token of the trace is a query row at least once (the row sources cover it)."""
    from tests.gpu_harness import schedule_trace
    from workloads import make_trace
    trace = make_trace("small", data_seed=11, n_spans=6, n_req=8, values=False)
    steps = schedule_trace(trace, policy, budget, max_running, num_blocks)
    replay(trace.span_lens, trace.requests, steps, policy, budget, num_blocks)
    src = np.concatenate([st["src"] for st in steps])
    assert np.array_equal(np.unique(src), np.arange(trace.n_tokens))
    for st in steps:
        assert st["src"].shape[0] == st["total_q"]


def test_trace_token_index():
    from workloads import make_trace
    t = make_trace("small", data_seed=11, n_spans=6, n_req=8, values=False)
    seen = []
    for s, n in enumerate(t.span_lens):
        seen.append(t.span_token_index(s, np.arange(n)))
    for r, (_, sids, p, o) in enumerate(t.requests):
        st = t.span_tokens(r)
        comp = t.request_token_index(r, np.arange(st + p + o))
        off = 0
        for s in sids:   # the spans' part maps onto the spans' own tokens
            assert np.array_equal(comp[off:off + t.span_lens[s]], t.span_token_index(s, np.arange(t.span_lens[s])))
            off += t.span_lens[s]
        seen.append(comp[st:])
    assert np.array_equal(np.sort(np.concatenate(seen)), np.arange(t.n_tokens))


def test_trace_oracle_first_tokens_are_their_values():
    """A span's first token and a span-less request's first private token see one key:
    the oracle output is that token's V, head group by head group."""
    import oracle
    from tests.oracle_harness import trace_token_outputs
    from workloads import make_trace
    t = make_trace("tiny", data_seed=3, n_spans=2, n_req=3, spans_per_req=(0, 1), hq=4, hkv=2,
                   d=16)
    firsts = [int(t.span_base[0])]
    firsts += [int(t.req_base[r]) for r, (_, sids, p, o) in enumerate(t.requests)
               if not sids and p + o > 0]
    out = trace_token_outputs(t, firsts)
    for n, g in enumerate(firsts):
        v = oracle.bf16_bits_to_f64(t.v[g])            # [Hkv][d]
        assert np.array_equal(out[n], np.repeat(v, t.hq // t.hkv, axis=0))

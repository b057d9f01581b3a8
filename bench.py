"""Benchmark: one serving step of position-free paged attention on one MI355X.

A step is the whole hot path over one batch: write the step's new (unrotated)
K/V into the paged cache (pic_cache_write), then one attention launch over
every request's context (pic_attn_decode for decode batches, pic_attn_prefill
for prefill / mixed batches).  The rotary table is built once at setup
(pic_rope_table) and timed separately.  Inputs are seeded synthetic data
resident in HBM before the timed region.

Default workload: 64 decode requests x (4096-token context + 1 new token),
Llama-3-8B layer shape (32 q / 8 kv heads, d 128, bf16), half of every
context in spans shared at different logical offsets.

Prints ONE JSON line on stdout; everything else goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix peak (256 CU x 4096 flop/clk x 2.4 GHz)
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X fp32 matrix peak

WORKLOAD_TEXT = {
    "c2": "decode 64 x (4096-token context + 1 new token), 2 of 4 1024-token segments shared "
          "spans, Llama-3-8B layer (32q/8kv, d128), bf16",
    "c2p": "decode 64 x (4096 + 1), all blocks private (control)",
    "c3": "chunked prefill 8 x (4 shared 1024-token spans + 512 causal suffix queries)",
    "c4": "long decode 4 x (131072-token context of 64 shared 2048-token spans + 1 new token)",
    "c5": "mixed single launch: 16 x 2048-token causal span prefills + 128 decodes of 8192+1",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source with comments and whitespace removed (string literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def source_hash() -> str:
    """Hash of the attention kernels' code (pic_attn.hip and the headers it includes,
    comments and whitespace removed): the traffic counters of the profiled kernels are only
    valid for this device code.  The other kernels' files and host-only C++ do not enter."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "position_independent_kv_amd", "csrc")
    for name in ["pic_attn.hip", "pic_common.hpp", "pic_device.hpp", "pic_host.hpp"]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def step_counts(w, counts):
    """Bytes of the whole step: attention's algorithmic bytes + the new tokens' K/V read+write."""
    es = 2 if w.dtype == "bf16" else 4
    cw = 2 * 2 * w.new_k.shape[0] * w.hkv * w.d * es + 4 * w.new_k.shape[0]
    return counts["bytes"] + cw


def pool_layers(w, cap=32):
    """Copies of a config's KV pools that the timed steps cycle through, as consecutive
    layers of one model would: at least 4, and enough for 1 GiB of pools (4x the 256 MB
    Infinity Cache), so every call finds the caches holding other layers' data."""
    es = 2 if w.dtype == "bf16" else 4
    pool = 2 * w.num_blocks * w.hkv * w.block_size * w.d * es
    return int(min(cap, max(4, -(-(1 << 30) // pool))))


def _event():
    """A timing event of the library (no system-scope fence at its records, which costs a
    step several microseconds with torch's default events)."""
    import position_independent_kv_amd as pic
    return pic.TimingEvent()


def _events(n):
    return [(_event(), _event()) for _ in range(n)]


def _ms(ev):
    return np.asarray([a.elapsed_time(b) for a, b in ev], np.float64)


def time_config(name, steps, warmup, with_rows=False, only_timed=False):
    """Time one config.  Timed region (the benchmark's K steps, after W warm-up steps):
    step k writes the new tokens into layer k's pools and runs the attention call on them,
    cycling over pool_layers(w) copies, so every call is cold (the Infinity Cache holds
    other layers' data).  A decode batch whose new tokens sit at each request's last key
    slot does both in one call (pic_attn_decode_append); other batches call
    pic_cache_write, then the attention.  The call's main kernel records HIP events at its
    start and end (pic_set_kernel_events; kernel_*: mean and median over the K steps), and
    events on the stream bracket the whole attention call in the same steps (call_*), so
    each step's kernel time lies inside its call time.  Unless only_timed, with >= 10
    warm-ups and >= 20 samples each: the cold call with no kernel events (what recording
    them costs); warm (one layer back to back): the main kernel and the call."""
    import torch

    import position_independent_kv_amd as pic
    from tests.gpu_harness import DeviceWorkload
    from workloads import algorithmic_counts, make_workload

    t = time.time()
    w = make_workload(name)
    counts = algorithmic_counts(w)
    nl = pool_layers(w)
    dw = DeviceWorkload(w).add_layers(nl)
    torch.cuda.synchronize()
    log(f"[bench] {name}: built in {time.time() - t:.1f}s; "
        f"{counts['bytes'] / 1e9:.3f} GB, {counts['flops'] / 1e12:.3f} TFLOP per attention call; "
        f"{nl} layer copies of the pools")
    stream = torch.cuda.current_stream()
    # A decode step writes its new tokens inside the decode launch (pic_attn_decode_append:
    # one launch fewer per step, same pool bytes and outputs); other steps write them with
    # pic_cache_write before the attention call.
    append = dw.appends_new_tokens()

    def pre():
        if not append:
            dw.write_new_tokens()

    def call():
        return dw.attention_append() if append else dw.attention()

    def loop(n, layer_of, hooked, first=0):
        """n steps; returns (kernel ms, call ms) per step (kernel None when not hooked)."""
        kev, cev = _events(n), _events(n)
        for k in range(n):
            dw.use_layer(layer_of(first + k))
            pre()
            if hooked:
                pic.pic_set_kernel_events(*kev[k])
            cev[k][0].record(stream)
            call()
            cev[k][1].record(stream)
        pic.pic_set_kernel_events(None, None)
        torch.cuda.synchronize()
        return (_ms(kev) if hooked else None), _ms(cev)

    def warm_up(n, layer_of):
        for k in range(n):
            dw.use_layer(layer_of(k))
            pre()
            call()

    warm_up(warmup, lambda k: k)
    kev, cev = _events(steps), _events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        dw.use_layer(warmup + k)
        pre()
        pic.pic_set_kernel_events(*kev[k])
        cev[k][0].record(stream)
        call()
        cev[k][1].record(stream)
    pic.pic_set_kernel_events(None, None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern, callt = _ms(kev), _ms(cev)
    # kernel and call of the same timed steps: the kernel's events lie inside the call's
    res = dict(name=name, w=w, counts=counts, layers=nl, appends=append,
               step_ms=(t1 - t0) * 1e3 / steps,
               kernel_ms=float(kern.mean()), kernel_median_ms=float(np.median(kern)),
               call_ms=float(callt.mean()), call_median_ms=float(np.median(callt)),
               step_bytes=step_counts(w, counts))
    if not only_timed:
        n, nw = max(20, steps), max(10, warmup)
        warm_up(nw, lambda k: k)
        _, plain = loop(n, lambda k: k, False)     # cold: the call alone, no kernel events
        warm_up(nw, lambda k: 0)
        wk, wc = loop(n, lambda k: 0, True)        # warm: one layer back to back
        res.update(call_unhooked_ms=float(np.median(plain)),
                   warm_kernel_ms=float(np.median(wk)), warm_call_ms=float(np.median(wc)),
                   samples=n, sample_warmup=nw)
    if with_rows and not only_timed:
        # the other rows of the path, timed on their own (same stream, events)
        stream = torch.cuda.current_stream()
        e = [_event() for _ in range(4)]
        cos = torch.empty_like(dw.cos)
        sin = torch.empty_like(dw.sin)
        e[0].record(stream)
        for _ in range(5):
            pic.pic_rope_table(cos, sin, w.base)
        e[1].record(stream)
        for _ in range(5):
            dw.write_new_tokens()
        e[2].record(stream)
        torch.cuda.synchronize()
        res["rope_table_ms"] = e[0].elapsed_time(e[1]) / 5
        res["cache_write_ms"] = e[1].elapsed_time(e[2]) / 5
        assert torch.equal(cos, dw.cos) and torch.equal(sin, dw.sin)
    del dw
    torch.cuda.empty_cache()
    return res


def rope_ablation(name, reps=20):
    """In-kernel rotation cost: position-free attention vs the same kernels over a
    conventional cache of pre-rotated keys (key rotation compiled out).

    Both calls read the same logical bytes and do the same matrix products; the
    rotated cache holds one private copy of every block per request (a shared span
    cannot be pre-rotated for two offsets).  Calls alternate, timed with HIP events
    on the launch stream.
    """
    import torch

    from tests.gpu_harness import DeviceWorkload
    from workloads import make_workload

    w = make_workload(name)
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    dw.build_rotated_cache()
    stream = torch.cuda.current_stream()
    for _ in range(10):
        dw.attention()
        dw.attention_rotated()
    torch.cuda.synchronize()
    ev = [[_event() for _ in range(4)] for _ in range(reps)]
    for k in range(reps):
        ev[k][0].record(stream)
        dw.attention()
        ev[k][1].record(stream)
        dw.attention_rotated()
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    pf = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    rot = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    res = {"workload": WORKLOAD_TEXT[name], "position_free_ms": pf, "rotated_cache_ms": rot,
           "rotation_overhead_frac": pf / rot - 1.0,
           "position_free_pool_blocks": int(w.num_blocks),
           "rotated_cache_pool_blocks": int(dw.rot_k_pool.shape[0])}
    log(f"[bench] rope ablation {name}: position-free {pf * 1e3:.1f} us, rotated cache "
        f"{rot * 1e3:.1f} us ({res['rotation_overhead_frac'] * 100:+.1f} %)")
    del dw
    torch.cuda.empty_cache()
    return res


def shared_decode(name, reps=20):
    """pic_attn_decode_shared against pic_attn_decode on one decode config: chunks cut
    where the blocks say and identical chunks side by side on one XCD, so shared spans are
    read once per XCD.  Calls alternate; main kernel (library-recorded events) and whole
    call (planning and merge launches included), medians of `reps`."""
    import torch

    import position_independent_kv_amd as pic
    from tests.gpu_harness import DeviceWorkload
    from workloads import algorithmic_counts, make_workload

    w = make_workload(name)
    counts = algorithmic_counts(w)
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    stream = torch.cuda.current_stream()
    calls = {"uniform_chunks": dw.attention, "shared_chunks": dw.attention_shared}
    for fn in calls.values():
        for _ in range(10):
            fn()
    torch.cuda.synchronize()
    ev = {k: [[_event() for _ in range(4)] for _ in range(reps)]
          for k in calls}
    for k in calls:
        for e in ev[k]:
            for x in e:
                x.record(stream)
    for i in range(reps):
        for k, fn in calls.items():
            e = ev[k][i]
            pic.pic_set_kernel_events(e[1], e[2])
            e[0].record(stream)
            fn()
            e[3].record(stream)
    pic.pic_set_kernel_events(None, None)
    torch.cuda.synchronize()
    res = {"workload": WORKLOAD_TEXT[name]}
    for k in calls:
        kern = float(np.median([e[1].elapsed_time(e[2]) for e in ev[k]]))
        call = float(np.median([e[0].elapsed_time(e[3]) for e in ev[k]]))
        res[k] = {"kernel_ms": kern, "call_ms": call,
                  "kernel_GBps": counts["bytes"] / (kern * 1e-3) / 1e9}
    res["kernel_speedup"] = res["uniform_chunks"]["kernel_ms"] / res["shared_chunks"]["kernel_ms"]
    res["call_speedup"] = res["uniform_chunks"]["call_ms"] / res["shared_chunks"]["call_ms"]
    log(f"[bench] shared decode {name}: main kernel {res['uniform_chunks']['kernel_ms'] * 1e3:.1f}"
        f" -> {res['shared_chunks']['kernel_ms'] * 1e3:.1f} us, call "
        f"{res['uniform_chunks']['call_ms'] * 1e3:.1f} -> {res['shared_chunks']['call_ms'] * 1e3:.1f} us")
    del dw
    torch.cuda.empty_cache()
    return res


def offload_bandwidth(n_blocks=4096, reps=5):
    """pic_blocks_copy between the device pools and a pinned host pool (CPU offload of
    position-free blocks): n_blocks whole blocks of the default layer shape (K+V = 64 KiB
    each in bf16), scattered ids, each direction timed with HIP events."""
    import torch

    import position_independent_kv_amd as pic
    shape_k, shape_v = (n_blocks, 8, 16, 128), (n_blocks, 8, 128, 16)
    dk = torch.randn(shape_k, device="cuda").to(torch.bfloat16)
    dv = torch.randn(shape_v, device="cuda").to(torch.bfloat16)
    hk = torch.empty(shape_k, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(shape_v, dtype=torch.bfloat16, pin_memory=True)
    rng = np.random.default_rng(3)
    src = torch.from_numpy(rng.permutation(n_blocks).astype(np.int32)).cuda()
    dst = torch.from_numpy(rng.permutation(n_blocks).astype(np.int32)).cuda()
    nbytes = 2 * dk.numel() * dk.element_size()
    stream = torch.cuda.current_stream()
    res = {}
    for label, args in [("device_to_host", (dk, dv, src, hk, hv, dst)),
                        ("host_to_device", (hk, hv, dst, dk, dv, src))]:
        pic.pic_blocks_copy(*args)
        torch.cuda.synchronize()
        e0, e1 = _event(), _event()
        e0.record(stream)
        for _ in range(reps):
            pic.pic_blocks_copy(*args)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[label] = {"ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9}
    ok = torch.equal(dk[src.long()].cpu(), hk[dst.long().cpu()])
    log(f"[bench] offload {n_blocks} blocks ({nbytes / 2**20:.0f} MiB): "
        f"d2h {res['device_to_host']['GBps']:.1f} GB/s, h2d {res['host_to_device']['GBps']:.1f} GB/s, "
        f"round trip exact: {ok}")
    res.update(blocks=n_blocks, bytes=nbytes, round_trip_exact=bool(ok))
    del dk, dv, hk, hv
    torch.cuda.empty_cache()
    return res


def scheduled_trace(budget=8192, max_running=32, num_blocks=8192, reps=3):
    """Interleaved span-prefill scheduling vs the barrier-separated policy on the RAG trace
    (64 requests in waves of 8, each 4 of 64 shared 1024-token spans + a 256-token final
    prompt + 32 output tokens): the library's scheduler builds every step's mixed batch,
    then each step is one cache write + one mixed attention launch.  Token values are drawn
    on the device.  Reports the attention-layer time of the whole trace (median of `reps`
    replays, HIP events around all steps) and the number of engine steps; a model's other
    layers (weights read once per step) are not part of this path."""
    import torch

    import position_independent_kv_amd as pic
    from tests.gpu_harness import TraceRun
    from workloads import RAG_TRACE, make_trace

    trace = make_trace(**{**RAG_TRACE, "values": False})
    res = {"trace": trace.description, "token_budget": budget, "max_running": max_running}
    stream = torch.cuda.current_stream()
    for label, policy in [("isps", pic.PIC_SCHED_ISPS), ("barrier", pic.PIC_SCHED_BARRIER)]:
        tr = TraceRun(trace, policy, budget, max_running, num_blocks, device_seed=5)
        tr.run()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = _event(), _event()
            e0.record(stream)
            tr.run()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        kinds = [len(set(st["seq_kind"].tolist())) for st in tr.steps if st["num_seqs"]]
        res[label] = {"attention_ms": ms, "steps": len(tr.steps),
                      "mixed_steps": int(sum(k > 1 for k in kinds)), "query_rows": tr.rows,
                      "requests_per_s": len(trace.requests) / (ms * 1e-3),
                      "query_rows_per_s": tr.rows / (ms * 1e-3)}
        log(f"[bench] scheduled trace {label}: {ms:.2f} ms over {len(tr.steps)} steps "
            f"({res[label]['mixed_steps']} mixed)")
        del tr
        torch.cuda.empty_cache()
    res["isps_speedup"] = res["barrier"]["attention_ms"] / res["isps"]["attention_ms"]
    res["isps_step_ratio"] = res["isps"]["steps"] / res["barrier"]["steps"]
    return res


def ceilings(reps=20):
    """What this GPU delivers outside the path: a plain streaming read (pic_stream_read over
    2 GiB, the best of a few grid sizes; medians of `reps`), a 2 GiB device copy (bytes read
    + written per second) and a large bf16 matrix product (torch.matmul, 8192^3)."""
    import torch

    import position_independent_kv_amd as pic
    nbytes = 2 << 30
    x = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")

    def stream_rate(wgs, order=None, piece=0):
        sink = torch.zeros(wgs * 256, dtype=torch.int32, device="cuda")
        for _ in range(3):
            pic.pic_stream_read(x, wgs, sink, order, piece)
        ev = _events(reps)
        for a, b in ev:
            a.record()
            pic.pic_stream_read(x, wgs, sink, order, piece)
            b.record()
        torch.cuda.synchronize()
        return nbytes / (float(np.median(_ms(ev))) * 1e-3) / 1e9

    read = {wgs: stream_rate(wgs) for wgs in (1024, 2048, 4096, 8192, 16384)}
    best = max(read, key=read.get)
    # the same bytes as randomly placed pieces: 4 KiB (one kv head of one 16-token bf16
    # block, d = 128), 16 KiB (four heads) and 32 KiB (a whole 8-head block)
    gather = {}
    for piece in (4096, 16384, 32768):
        perm = np.random.default_rng(9).permutation(nbytes // piece).astype(np.int32)
        order = torch.from_numpy(perm).cuda()
        gather[str(piece)] = max(stream_rate(wgs, order, piece) for wgs in (2048, 8192))
        del order
    y = torch.empty_like(x)
    y.copy_(x)
    ev = _events(reps)
    for a, b in ev:
        a.record()
        y.copy_(x)
        b.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes / (float(np.median(_ms(ev))) * 1e-3) / 1e9
    del x, y
    n = 8192
    a_ = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b_ = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = a_ @ b_
    ev = _events(10)
    for a, b in ev:
        a.record()
        c = a_ @ b_
        b.record()
    torch.cuda.synchronize()
    mm_tflops = 2 * n ** 3 / (float(np.median(_ms(ev))) * 1e-3) / 1e12
    del a_, b_, c
    torch.cuda.empty_cache()
    log(f"[bench] ceilings: streaming read {read[best]:.0f} GB/s ({best} workgroups), random "
        f"4/16/32 KiB pieces {gather['4096']:.0f}/{gather['16384']:.0f}/{gather['32768']:.0f} "
        f"GB/s, device copy {copy_gbps:.0f} GB/s, bf16 matmul {mm_tflops:.0f} TFLOP/s")
    return {"stream_read_GBps": read[best], "stream_read_workgroups": best,
            "stream_read_sweep_GBps": {str(k): v for k, v in read.items()},
            "gather_read_GBps_by_piece_bytes": gather,
            "device_copy_GBps": copy_gbps, "bf16_matmul_TFLOPs": mm_tflops,
            "note": "pic_stream_read over 2 GiB (16-byte loads, 8 per lane in flight, best grid), "
                    "front to back and as randomly ordered pieces; "
                    "2 GiB torch copy (read + write bytes); torch.matmul bf16 8192^3; medians"}


def attention_ceiling(reps=20):
    """This GPU's library dense attention at the chunked-prefill shape, for context: torch's
    scaled_dot_product_attention restricted to its flash backend (no fallback to a math
    path), bf16, 8 requests x 32 heads x 512 queries over 4608 keys (kv heads expanded
    to 32, keys already rotated: no paging, no positions), dense and with the
    bottom-right causal mask.  Flops counted as for the path: 4 d per unmasked
    (query, key, head)."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    from torch.nn.attention.bias import causal_lower_right
    B, H, Tq, Tk, d = 8, 32, 512, 4608, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    q = torch.randn((B, H, Tq, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, H, Tk, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, Tk, d), generator=g, device="cuda").to(torch.bfloat16)
    res = {"shape": f"{B} x {H} heads x {Tq} queries x {Tk} keys, d {d}, bf16"}
    pairs = {"dense": Tq * Tk, "causal_lower_right": Tq * (Tk - Tq) + Tq * (Tq + 1) // 2}
    for label, mask in [("dense", None), ("causal_lower_right", causal_lower_right(Tq, Tk))]:
        try:
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
                torch.cuda.synchronize()
                ev = _events(reps)
                for a, b in ev:
                    a.record()
                    torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
                    b.record()
                torch.cuda.synchronize()
            ms = float(np.median(_ms(ev)))
            res[label] = {"ms": ms, "TFLOPs": 4 * d * B * H * pairs[label] / (ms * 1e-3) / 1e12}
        except Exception as e:  # the flash backend of this torch version may not take this mask
            res[label] = {"error": f"{type(e).__name__}: {str(e)[:160]}"}
    del q, k, v
    torch.cuda.empty_cache()
    log(f"[bench] attention ceiling (torch SDPA flash): {res}")
    return res


def prefill_scaling(lengths=(512, 1024, 2048, 4096, 8192, 16384), reps=10):
    """One causal span prefill alone (q_len = seq_len = N, positions 0..N-1, the span
    written by the step) at growing N: the mixed launch's main kernel time and TFLOP/s
    (medians of `reps` after 3 warm-ups, warm), the kernel-level counterpart of prefill
    time growing with the span length."""
    import torch

    import position_independent_kv_amd as pic
    from tests.gpu_harness import DeviceWorkload
    from workloads import algorithmic_counts, make_workload
    res = {}
    for n in lengths:
        w = make_workload(f"span{n}", builder="mixed", seed=7, n_chunks=1, chunk=n, n_dec=0,
                          per_dec=0)
        c = algorithmic_counts(w)
        dw = DeviceWorkload(w)
        dw.write_new_tokens()
        for _ in range(3):
            dw.attention()
        ev = _events(reps)
        for a, b in ev:
            pic.pic_set_kernel_events(a, b)
            dw.attention()
        pic.pic_set_kernel_events(None, None)
        torch.cuda.synchronize()
        ms = float(np.median(_ms(ev)))
        res[str(n)] = {"kernel_ms": ms, "TFLOPs": c["flops"] / (ms * 1e-3) / 1e12,
                       "flops": c["flops"]}
        del dw
        torch.cuda.empty_cache()
    log("[bench] prefill scaling (one causal span): " +
        ", ".join(f"{k}: {v['kernel_ms'] * 1e3:.0f} us {v['TFLOPs']:.0f} TF/s" for k, v in res.items()))
    return res


def block_table_build(reps=5):
    """Host cost of the span-aware block tables (pic_build_block_tables) for a batch
    composed like the default decode workload: 64 prompts of 4 x 1024 tokens, two of
    them SSEP spans drawn from a pool of 32 (so shared), two private, each prompt
    closed by a 16-token PDEP block.  Median of `reps` builds."""
    import position_independent_kv_amd as pic
    rng = np.random.default_rng(7)
    ssep, pdep = 128001, 128002
    spans = [np.concatenate([[ssep], rng.integers(0, 120000, 1023)]).astype(np.int32)
             for _ in range(32)]
    prompts = []
    for _ in range(64):
        k = rng.choice(32, size=2, replace=False)
        own = [rng.integers(0, 120000, 1024).astype(np.int32) for _ in range(2)]
        suffix = np.concatenate([[pdep], rng.integers(0, 120000, 15)]).astype(np.int32)
        prompts.append(np.concatenate([own[0], spans[k[0]], own[1], spans[k[1]], suffix]))
    toks = np.concatenate(prompts)
    cu = np.concatenate([[0], np.cumsum([len(p) for p in prompts])]).astype(np.int32)
    times = []
    for _ in range(reps):
        t = time.perf_counter()
        res = pic.pic_build_block_tables(toks, cu, 16, ssep, pdep, seed=1)
        times.append(time.perf_counter() - t)
    ms = float(np.median(times)) * 1e3
    logical = int(sum(-(-len(p) // 16) for p in prompts))
    log(f"[bench] block tables: {toks.shape[0]} tokens in {ms:.2f} ms on the host; "
        f"{res['num_new_blocks']} physical blocks for {logical} logical")
    return {"tokens": int(toks.shape[0]), "host_ms": ms,
            "tokens_per_s": toks.shape[0] / (ms * 1e-3),
            "physical_blocks": res["num_new_blocks"], "logical_blocks": logical}


def request_work(w):
    """Per request: the algorithmic bytes attention must move for it (K and V of its
    visible slots, its q and out rows, its metadata) and its flops (4 d per unmasked
    (row, key, q head)).  The cos/sin table is shared by the batch and not split."""
    es = 2 if w.dtype == "bf16" else 4
    ql = w.q_lens().astype(np.float64)
    L = w.seq_lens.astype(np.float64)
    byts = (L * w.hkv * w.d * es * 2 + 2 * ql * w.hq * w.d * es
            + 4 * (np.ceil(L / w.block_size) + L + ql + 2))
    pairs = ql * (L - ql) + ql * (ql + 1) / 2
    return byts, 4.0 * w.d * w.hq * pairs


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def oracle_rate(w, counts, budget_s, unit, threads=None):
    """The fp64 oracle (as it is, untuned) on the host over the first n requests of the
    config, n chosen so the sample takes about budget_s (at least one request), repeated
    while the measured time stays under budget_s (at most 8 runs).  Returns the rate in
    `unit` ("GB/s": the sample's share of the call's algorithmic bytes; "TFLOP/s": the
    sample's flops) and the sample's description."""
    import contextlib

    import oracle
    from tests.oracle_harness import oracle_pools
    kp, vp = oracle_pools(w)

    def run(reqs):
        t = time.perf_counter()
        oracle.attention(w.q, w.cu_seqlens_q, w.q_pos, kp, vp, w.block_table, w.seq_lens,
                         w.cu_seqlens_k, w.k_pos, w.base, w.block_size, requests=reqs)
        return time.perf_counter() - t

    ctx = contextlib.nullcontext()
    if threads is not None:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(threads)
    with ctx:
        nthreads = _blas_threads()
        t1 = run([0])
        n = int(max(1, min(w.num_reqs, budget_s / max(t1, 1e-6))))
        reqs = list(range(n))
        dt, reps = (t1, 1) if n == 1 else (0.0, 0)
        while reps == 0 or (dt < budget_s and reps < 8):
            dt += run(reqs)
            reps += 1
    rb, rf = request_work(w)
    if unit == "GB/s":
        work = counts["bytes"] * rb[:n].sum() / rb.sum() / 1e9
    else:
        work = rf[:n].sum() / 1e12
    return {"value": work * reps / dt, "unit": unit, "cores": nthreads, "kind": "oracle",
            "sample": f"first {n} of {w.num_reqs} requests of the {w.name} attention call, "
                      f"{reps} run(s), {dt:.1f} s, numpy fp64, {nthreads} BLAS threads"}


def cpu_model():
    cpu = os.popen("lscpu 2>/dev/null | grep 'Model name' | head -1").read()
    return " ".join(cpu.split(":", 1)[-1].split())


def config_unit(w):
    return "GB/s" if w.kind == "decode" else "TFLOP/s"


def load_traffic(kernel: str, config: str):
    """HBM bytes per launch of `kernel` (the call's main kernel) from the committed
    rocprofv3 --pmc summaries, if still valid for the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        data = json.load(f)
    ent = data.get(kernel + ":" + config)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    part = ent.get("parts", {}).get(kernel)
    return part["bytes"] if part else None


def copy_calibration(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling the PMC byte counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {nbytes} bytes")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--others", default="c2p,c3,c4,c5",
                    help="comma list of further configs reported under 'configs' ('' for none)")
    ap.add_argument("--ablation", default="c2p,c3,c4",
                    help="configs on which to time the in-kernel rotation ablation ('' for none)")
    ap.add_argument("--shared", default="c2,c4",
                    help="decode configs on which to compare pic_attn_decode_shared ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sched", action="store_true",
                    help="skip the scheduled-trace comparison (ISPS vs barrier)")
    ap.add_argument("--only-main", action="store_true",
                    help="only the headline config's timed region (profiling runs: the kernel "
                         "averages rocprofv3 reports are then those of the timed steps)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="only run a plain copy of this many bytes (PMC scaling run)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path "
              "shards by request and kv head with no exchange, so one GPU's share is what is "
              "measured)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return
    if args.only_main:
        args.others = args.ablation = args.shared = ""
        args.no_cpu_baseline = args.no_sched = True

    main_res = time_config(args.config, args.steps, args.warmup, with_rows=True,
                           only_timed=args.only_main)
    w, counts = main_res["w"], main_res["counts"]
    if not args.only_main:
        m = main_res
        log(f"[bench] {args.config}: timed steps (cold, means): kernel {m['kernel_ms'] * 1e3:.1f} us "
            f"within call {m['call_ms'] * 1e3:.1f} us; call without kernel events "
            f"{m['call_unhooked_ms'] * 1e3:.1f} us; warm kernel {m['warm_kernel_ms'] * 1e3:.1f} us")
    decode = w.kind == "decode"
    kernel = "decode_kernel" if decode else "mixed_kernel"
    if decode:
        work, scale, peak, unit = counts["bytes"], 1e9, HBM_PEAK_GBS, "GB/s"
        roof = {"bound": "hbm"}
        value = main_res["step_bytes"] / (main_res["step_ms"] * 1e-3) / 1e9
        metric = "decode HBM GB/s"
    else:
        work, scale, unit = counts["flops"], 1e12, "TFLOP/s"
        peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
        roof = {"bound": "mfma"}
        value = counts["flops"] / (main_res["step_ms"] * 1e-3) / 1e12
        metric = "prefill TFLOP/s"

    def rate(ms):
        return work / (ms * 1e-3) / scale

    achieved = rate(main_res["kernel_ms"])
    roof.update(achieved=achieved, peak=peak, unit=unit, frac=achieved / peak,
                traffic=load_traffic(kernel, args.config), kernel=kernel,
                timing="cold: the timed steps cycle over %d copies of the KV pools (layers), so "
                       "no call finds its data in the caches; achieved = algorithmic work / mean "
                       "main-kernel time over the timed steps (events recorded by the kernel's "
                       "dispatch)%s" % (main_res["layers"],
                                        "; each step's new tokens are written by the decode "
                                        "launch itself (pic_attn_decode_append)"
                                        if main_res["appends"] else
                                        "; each step writes its new tokens with "
                                        "pic_cache_write, then runs the attention call"),
                kernel_ms=main_res["kernel_ms"], kernel_median_ms=main_res["kernel_median_ms"],
                algorithmic_bytes=counts["bytes"], algorithmic_flops=counts["flops"],
                unique_kv_bytes=counts["unique_kv_bytes"])
    if "warm_kernel_ms" in main_res:
        roof.update(call_ms=main_res["call_ms"], call_median_ms=main_res["call_median_ms"],
                    call_frac=rate(main_res["call_ms"]) / peak,
                    call_unhooked_ms=main_res["call_unhooked_ms"],
                    warm_kernel_ms=main_res["warm_kernel_ms"],
                    warm_frac=rate(main_res["warm_kernel_ms"]) / peak,
                    warm_call_ms=main_res["warm_call_ms"],
                    samples=main_res["samples"], sample_warmup=main_res["sample_warmup"])

    cpu = None
    per_cfg = {}
    if not args.no_cpu_baseline:
        from workloads import make_workload
        t = time.time()
        cpu = oracle_rate(w, counts, 12.0, unit)
        cpu["cpu"] = cpu_model()
        cpu["single_core"] = oracle_rate(w, counts, 6.0, unit, threads=1)
        c1 = make_workload("c1a")
        from workloads import algorithmic_counts
        c1c = algorithmic_counts(c1)
        per_cfg["c1a"] = oracle_rate(c1, c1c, 2.0, "TFLOP/s")
        per_cfg["c1a"]["single_core"] = oracle_rate(c1, c1c, 2.0, "TFLOP/s", threads=1)
        log(f"[bench] cpu baseline {args.config} + c1a in {time.time() - t:.1f}s: "
            f"{cpu['value']:.4g} {unit}")

    others = {}
    for name in [x for x in args.others.split(",") if x]:
        if name == args.config:
            continue
        r = time_config(name, max(20, args.steps), max(10, args.warmup))
        c = r["counts"]
        others[name] = {
            "workload": WORKLOAD_TEXT[name], "layers": r["layers"],
            "kernel_ms": r["kernel_ms"], "kernel_median_ms": r["kernel_median_ms"],
            "call_ms": r["call_ms"], "call_median_ms": r["call_median_ms"],
            "call_unhooked_ms": r["call_unhooked_ms"],
            "warm_kernel_ms": r["warm_kernel_ms"],
            "warm_call_ms": r["warm_call_ms"], "step_ms": r["step_ms"],
            "samples": r["samples"],
            "kernel_GBps": c["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9,
            "kernel_hbm_frac": c["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernel_TFLOPs": c["flops"] / (r["kernel_ms"] * 1e-3) / 1e12,
            "kernel_mfma_frac": c["flops"] / (r["kernel_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "call_GBps": c["bytes"] / (r["call_ms"] * 1e-3) / 1e9,
            "call_TFLOPs": c["flops"] / (r["call_ms"] * 1e-3) / 1e12,
            "warm_kernel_GBps": c["bytes"] / (r["warm_kernel_ms"] * 1e-3) / 1e9,
            "warm_kernel_TFLOPs": c["flops"] / (r["warm_kernel_ms"] * 1e-3) / 1e12,
            "unique_kv_bytes": c["unique_kv_bytes"], "algorithmic_bytes": c["bytes"],
            "flops": c["flops"],
        }
        log(f"[bench] {name}: timed steps (cold, means): kernel {r['kernel_ms'] * 1e3:.1f} us "
            f"within call {r['call_ms'] * 1e3:.1f} us; call without kernel events "
            f"{r['call_unhooked_ms'] * 1e3:.1f} us; warm kernel {r['warm_kernel_ms'] * 1e3:.1f} us; "
            f"{others[name]['kernel_GBps']:.0f} GB/s, {others[name]['kernel_TFLOPs']:.1f} TFLOP/s")
        if not args.no_cpu_baseline:
            t = time.time()
            per_cfg[name] = oracle_rate(r["w"], c, 20.0 if name == "c4" else 6.0,
                                        config_unit(r["w"]))
            log(f"[bench] cpu baseline {name} in {time.time() - t:.1f}s: "
                f"{per_cfg[name]['value']:.4g} {per_cfg[name]['unit']}")
        del r
    if cpu is not None:
        cpu["per_config"] = per_cfg

    ablation = {}
    for name in [x for x in args.ablation.split(",") if x]:
        ablation[name] = rope_ablation(name)
    shared = {}
    for name in [x for x in args.shared.split(",") if x]:
        shared[name] = shared_decode(name)
    tables = block_table_build() if not args.only_main else None
    sched = None if args.no_sched else scheduled_trace()
    ceil = ceilings() if not args.only_main else None
    if ceil is not None:
        ceil["attention"] = attention_ceiling()
    scaling = prefill_scaling() if not args.only_main else None
    offload = offload_bandwidth() if not args.only_main else None

    out = {
        "metric": f"position-free paged attn: {metric}",
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) K/V/q; no dataset or weights)",
        "config": {"workload": WORKLOAD_TEXT[args.config], "name": args.config,
                   "requests": w.num_reqs, "query_rows": w.total_q,
                   "max_seq_len": w.max_seq_len, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.d, "block_size": w.block_size, "rope_base": w.base,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "rows": {"rope_table_ms": main_res.get("rope_table_ms"),
                 "cache_write_ms": main_res.get("cache_write_ms"),
                 "attention_call_ms": main_res.get("call_unhooked_ms"),
                 "attention_kernel_ms": main_res["kernel_ms"]},
        "configs": others,
        "rope_ablation": ablation,
        "shared_decode": shared,
        "block_tables": tables,
        "scheduled_trace": sched,
        "ceilings": ceil,
        "prefill_scaling": scaling,
        "offload": offload,
        "source_hash": source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

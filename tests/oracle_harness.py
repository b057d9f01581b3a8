"""Oracle plumbing for tests: the fp64 reference over a Workload (CPU only)."""

from __future__ import annotations

import numpy as np

import oracle
from workloads import Workload


# ---------------------------------------------------------------------------
# oracle side
# ---------------------------------------------------------------------------

def oracle_pools(w: Workload):
    """The pools as the cache holds them after the step's writes (oracle placement)."""
    sdt = np.uint16 if w.dtype == "bf16" else np.float32
    B = w.block_size
    kp = np.zeros((w.num_blocks, w.hkv, B, w.d), sdt)
    vp = np.zeros((w.num_blocks, w.hkv, w.d, B), sdt)
    if w.ctx_k.shape[0]:
        oracle.place_tokens(w.ctx_k, w.ctx_v, w.ctx_slots, kp, vp, B)
    oracle.place_tokens(w.new_k, w.new_v, w.new_slots, kp, vp, B)
    return kp, vp


def oracle_outputs(w: Workload, requests=None, rows=None, pools=None) -> np.ndarray:
    """fp64 reference rows, concatenated in (request, row) order."""
    kp, vp = oracle_pools(w) if pools is None else pools
    res = oracle.attention(w.q, w.cu_seqlens_q, w.q_pos, kp, vp, w.block_table, w.seq_lens,
                           w.cu_seqlens_k, w.k_pos, w.base, w.block_size, requests=requests,
                           rows=rows)
    keys = list(res.keys()) if requests is None else list(requests)
    return np.concatenate([res[r] for r in keys], axis=0)


def select_rows(out: np.ndarray, w: Workload, requests, rows=None) -> np.ndarray:
    """Pick the GPU output rows matching oracle_outputs(w, requests, rows)."""
    parts = []
    for r in requests:
        q0 = int(w.cu_seqlens_q[r])
        ql = int(w.cu_seqlens_q[r + 1]) - q0
        sel = np.arange(ql) if rows is None or r not in rows else np.asarray(rows[r])
        parts.append(out[q0 + sel])
    return np.concatenate(parts, axis=0)


def trace_token_outputs(trace, tokens) -> np.ndarray:
    """fp64 reference output of each listed token of a scheduled trace, [n][Hq][d].

    A span token i of span s attends to tokens 0..i of that span at positions
    0..i (a span is prefilled on its own); a request's private token at
    composed slot c attends to slots 0..c of the request's composed sequence
    (its spans in order, then its private tokens) at positions 0..c.  The
    output does not depend on how a schedule batches or chunks the work.
    One oracle call per span or request covers all its listed tokens.
    """
    tokens = np.asarray(tokens, np.int64)
    out = np.zeros((tokens.shape[0], trace.hq, trace.d))
    n_span_tok = int(sum(trace.span_lens))
    span_end = np.asarray(trace.span_base) + np.asarray(trace.span_lens)
    groups = {}
    for n, g in enumerate(tokens):
        if g < n_span_tok:
            s = int(np.searchsorted(span_end, g, side="right"))
            groups.setdefault(("span", s), []).append((n, int(g - trace.span_base[s])))
        else:
            # the last request starting at or before g (requests without private
            # tokens share their successor's base and are passed over)
            r = int(np.searchsorted(trace.req_base, g, side="right")) - 1
            c = int(g - trace.req_base[r]) + trace.span_tokens(r)
            groups.setdefault(("req", r), []).append((n, c))
    for (kind, i), items in groups.items():
        slots = np.array([c for _, c in items])
        L = int(slots.max()) + 1
        first = 0 if kind == "span" else trace.span_tokens(i)  # first query slot
        idx = (trace.span_token_index(i, np.arange(L)) if kind == "span"
               else trace.request_token_index(i, np.arange(L)))
        q_slots = np.arange(first, L)
        res = oracle.attention_request(trace.q[idx[q_slots]], q_slots, trace.k[idx],
                                       trace.v[idx], np.arange(L), L - first, trace.base,
                                       trace.hkv, rows=slots - first)
        for (n, _), row in zip(items, res):
            out[n] = row
    return out

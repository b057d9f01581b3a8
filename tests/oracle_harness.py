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

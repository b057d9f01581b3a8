"""Test-side plumbing: run a Workload through the HIP library, or through the oracle.

The GPU side only calls the C ABI through the Python binding; the oracle side
only calls ``oracle/``.  Both consume the same ``workloads`` arrays.
"""

from __future__ import annotations

import numpy as np

import oracle
import position_independent_kv_amd as pic
from workloads import Workload


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def to_torch(a: np.ndarray, dtype: str, dev="cuda"):
    """Stored values (uint16 bf16 bits or float32) -> torch tensor on dev."""
    torch = _torch()
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a.astype(np.float32)).to(dev)


def i32(a, dev="cuda"):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class DeviceWorkload:
    """A Workload resident on the GPU: metadata, q, table, pools (context written)."""

    def __init__(self, w: Workload, dev="cuda", fill=float("nan"), write_context=True):
        torch = _torch()
        self.w = w
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.dtype = tdt
        self.q = to_torch(w.q, w.dtype, dev)
        self.cu_q = i32(w.cu_seqlens_q, dev)
        self.q_pos = i32(w.q_pos, dev)
        self.block_table = i32(w.block_table, dev)
        self.seq_lens = i32(w.seq_lens, dev)
        self.cu_k = i32(w.cu_seqlens_k, dev)
        self.k_pos = i32(w.k_pos, dev)
        B = w.block_size
        # pools start as NaN: any read of a slot that was never written shows up
        self.k_pool = torch.full((w.num_blocks, w.hkv, B, w.d), fill, dtype=tdt, device=dev)
        self.v_pool = torch.full((w.num_blocks, w.hkv, w.d, B), fill, dtype=tdt, device=dev)
        self.cos = torch.empty((w.max_pos, w.d // 2), dtype=torch.float32, device=dev)
        self.sin = torch.empty_like(self.cos)
        pic.pic_rope_table(self.cos, self.sin, w.base)
        self.new_k = to_torch(w.new_k, w.dtype, dev)
        self.new_v = to_torch(w.new_v, w.dtype, dev)
        self.new_slots = i32(w.new_slots, dev)
        if write_context and w.ctx_k.shape[0]:
            pic.pic_cache_write(to_torch(w.ctx_k, w.dtype, dev), to_torch(w.ctx_v, w.dtype, dev),
                                i32(w.ctx_slots, dev), self.k_pool, self.v_pool)
        self.out = torch.empty_like(self.q)
        ws = pic.pic_attn_workspace_size(w.num_reqs, w.total_q, w.max_seq_len, w.hq, w.hkv, w.d,
                                         tdt)
        self.workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=dev)

    def write_new_tokens(self):
        if self.new_slots.shape[0]:
            pic.pic_cache_write(self.new_k, self.new_v, self.new_slots, self.k_pool, self.v_pool)

    def attention(self, decode=None, out=None):
        w = self.w
        out = self.out if out is None else out
        if decode is None:
            decode = w.kind == "decode"
        if decode:
            pic.pic_attn_decode(self.q, self.q_pos, self.k_pool, self.v_pool, self.block_table,
                                self.seq_lens, self.cu_k, self.k_pos, self.cos, self.sin,
                                w.max_seq_len, out, self.workspace)
        else:
            pic.pic_attn_prefill(self.q, self.cu_q, self.q_pos, self.k_pool, self.v_pool,
                                 self.block_table, self.seq_lens, self.cu_k, self.k_pos, self.cos,
                                 self.sin, w.max_q_len, w.max_seq_len, out, self.workspace)
        return out

    def step(self, decode=None):
        """One serving step: write the new tokens, then attention."""
        self.write_new_tokens()
        return self.attention(decode)


def run_workload(w: Workload, decode=None) -> np.ndarray:
    torch = _torch()
    dw = DeviceWorkload(w)
    out = dw.step(decode)
    torch.cuda.synchronize()
    return to_f64(out)


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

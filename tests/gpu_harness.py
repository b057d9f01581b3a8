"""GPU plumbing for tests and the benchmark: run a Workload through the HIP library.

Only calls the C ABI through the Python binding; never touches ``oracle/``
(the oracle side lives in ``tests/oracle_harness.py``).  Both sides consume
the same ``workloads`` arrays.
"""

from __future__ import annotations

import numpy as np

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
        # outputs start as NaN too: a row that no kernel writes fails every comparison
        self.out = torch.full_like(self.q, float("nan"))
        ws = pic.pic_attn_workspace_size(w.num_reqs, w.total_q, w.max_seq_len, w.hq, w.hkv, w.d,
                                         tdt)
        self.workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=dev)

    def add_layers(self, n):
        """n - 1 further copies of the pools, standing for the KV caches of other layers of one
        model (same blocks, same metadata); use_layer(i) points the calls at copy i % n."""
        self.layers = [(self.k_pool, self.v_pool)]
        self.layers += [(self.k_pool.clone(), self.v_pool.clone()) for _ in range(n - 1)]
        return self

    def use_layer(self, i):
        self.k_pool, self.v_pool = self.layers[i % len(self.layers)]

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

    def attention_shared(self, out=None):
        """The batch through pic_attn_decode_shared (block-determined chunks, identical
        chunks side by side on one XCD); its workspace is allocated on first use."""
        w = self.w
        out = self.out if out is None else out
        if getattr(self, "shared_ws", None) is None:
            n = pic.pic_attn_decode_shared_workspace_size(w.num_reqs, w.max_seq_len, w.hq, w.hkv,
                                                          w.d, self.dtype)
            self.shared_ws = _torch().zeros(max(n, 16), dtype=_torch().uint8, device=out.device)
        pic.pic_attn_decode_shared(self.q, self.q_pos, self.k_pool, self.v_pool,
                                   self.block_table, self.seq_lens, self.cu_k, self.k_pos,
                                   self.cos, self.sin, w.max_seq_len, out, self.shared_ws)
        return out

    def build_rotated_cache(self):
        """The conventional RoPE cache of this batch, for the in-kernel-rotation ablation.

        Every request gets private blocks holding its own slots' keys rotated to
        its own positions (pic_cache_write_rotated); a shared span is therefore
        stored once per request that uses it.  Reads the pools as they are now
        (call after the step's cache write).  Sets rot_k_pool, rot_v_pool and
        rot_block_table.
        """
        torch = _torch()
        w = self.w
        B = w.block_size
        L = w.seq_lens.astype(np.int64)
        nblk = (L + B - 1) // B
        base = np.concatenate([[0], np.cumsum(nblk)[:-1]]).astype(np.int64)
        total = int(nblk.sum())
        stride = max(int(nblk.max()) if len(nblk) else 1, 1)
        bt = np.zeros((w.num_reqs, stride), np.int32)
        src, dst, pos = [], [], []
        for r in range(w.num_reqs):
            j = np.arange(int(L[r]), dtype=np.int64)
            bt[r, :nblk[r]] = base[r] + np.arange(nblk[r])
            src.append(w.block_table[r, j // B].astype(np.int64) * B + j % B)
            dst.append((base[r] + j // B) * B + j % B)
            pos.append(w.k_pos[int(w.cu_seqlens_k[r]):int(w.cu_seqlens_k[r]) + int(L[r])])
        src = np.concatenate(src) if src else np.zeros(0, np.int64)
        dst = np.concatenate(dst) if dst else np.zeros(0, np.int64)
        pos = np.concatenate(pos) if pos else np.zeros(0, np.int32)
        dev = self.k_pool.device
        s_t = torch.from_numpy(src).to(dev)
        blk, off = s_t // B, s_t % B
        k_tok = self.k_pool[blk, :, off, :].contiguous()      # [T][Hkv][d]
        v_tok = self.v_pool[blk, :, :, off].contiguous()      # [T][Hkv][d]
        self.rot_k_pool = torch.full((max(total, 1), w.hkv, B, w.d), float("nan"),
                                     dtype=self.dtype, device=dev)
        self.rot_v_pool = torch.full((max(total, 1), w.hkv, w.d, B), float("nan"),
                                     dtype=self.dtype, device=dev)
        self.rot_block_table = i32(bt, dev)
        if src.shape[0]:
            pic.pic_cache_write_rotated(k_tok, v_tok, i32(dst, dev), i32(pos, dev), self.cos,
                                        self.sin, self.rot_k_pool, self.rot_v_pool)
        return self

    def attention_rotated(self, decode=None, out=None):
        """The same attention over the rotated cache (key rotation compiled out)."""
        w = self.w
        out = self.out if out is None else out
        if decode is None:
            decode = w.kind == "decode"
        if decode:
            pic.pic_attn_decode_rotated(self.q, self.q_pos, self.rot_k_pool, self.rot_v_pool,
                                        self.rot_block_table, self.seq_lens, self.cos, self.sin,
                                        w.max_seq_len, out, self.workspace)
        else:
            pic.pic_attn_prefill_rotated(self.q, self.cu_q, self.q_pos, self.rot_k_pool,
                                         self.rot_v_pool, self.rot_block_table, self.seq_lens,
                                         self.cos, self.sin, w.max_q_len, w.max_seq_len, out,
                                         self.workspace)
        return out

    def step(self, decode=None):
        """One serving step: write the new tokens, then attention."""
        self.write_new_tokens()
        return self.attention(decode)

    def appends_new_tokens(self) -> bool:
        """Whether the batch's new tokens are one per request, in request order, each at its
        request's last key slot (what pic_attn_decode_append writes)."""
        w = self.w
        if w.kind != "decode" or w.new_slots.shape[0] != w.num_reqs:
            return False
        L = np.asarray(w.seq_lens, np.int64)
        if (L < 1).any():
            return False
        bt = np.asarray(w.block_table, np.int64)
        last = bt[np.arange(w.num_reqs), (L - 1) // w.block_size] * w.block_size \
            + (L - 1) % w.block_size
        return bool(np.array_equal(last, np.asarray(w.new_slots, np.int64)))

    def attention_append(self, out=None):
        """A decode step in one call: the decode launch writes request r's new token (row r
        of new_k / new_v, its key slot seq_lens[r] - 1) itself (pic_attn_decode_append)."""
        w = self.w
        out = self.out if out is None else out
        pic.pic_attn_decode_append(self.q, self.new_k, self.new_v, self.q_pos, self.k_pool,
                                   self.v_pool, self.block_table, self.seq_lens, self.cu_k,
                                   self.k_pos, self.cos, self.sin, w.max_seq_len, out,
                                   self.workspace)
        return out


def run_workload(w: Workload, decode=None) -> np.ndarray:
    torch = _torch()
    dw = DeviceWorkload(w)
    out = dw.step(decode)
    torch.cuda.synchronize()
    return to_f64(out)


# ---------------------------------------------------------------------------
# scheduled traces (interleaved span-prefill scheduling)
# ---------------------------------------------------------------------------

def schedule_trace(trace, policy: int, budget: int, max_running: int, num_blocks: int):
    """Run the library's scheduler over a trace (host).  Returns the steps, each the
    pic_sched_step dict plus ``src``: the global token index of every query row."""
    B = pic.BLOCK_SIZE
    R = len(trace.requests)
    max_len = max([trace.composed_len(r) for r in range(R)] + list(trace.span_lens))
    stride = -(-max_len // B)
    max_seqs = max_running + len(trace.span_lens)
    sched = pic.Scheduler(policy, budget, max_running, num_blocks, max_seqs=max_seqs,
                          max_keys=max_seqs * max_len, block_table_stride=stride)
    try:
        for n in trace.span_lens:
            sched.add_span(n)
        for (arr, sids, p, o) in trace.requests:
            sched.add_request(arr, sids, p, o)
        steps = []
        while True:
            st = sched.step()
            if st is None:
                break
            src = []
            for i in range(st["num_seqs"]):
                kind, sid, qb = int(st["seq_kind"][i]), int(st["seq_id"][i]), int(st["q_begin"][i])
                ql = int(st["cu_seqlens_q"][i + 1] - st["cu_seqlens_q"][i])
                c = np.arange(qb, qb + ql)
                src.append(trace.span_token_index(sid, c) if kind == pic.PIC_SEQ_SPAN
                           else trace.request_token_index(sid, c))
            st["src"] = np.concatenate(src) if src else np.zeros(0, np.int64)
            steps.append(st)
    finally:
        sched.close()
    return steps


class TraceRun:
    """A scheduled trace staged on the GPU: every step's q/k/v rows and metadata resident,
    then ``run()`` enqueues the steps (cache write + one mixed attention launch each)."""

    def __init__(self, trace, policy: int, budget: int, max_running: int, num_blocks: int,
                 dev="cuda", device_seed=None):
        """device_seed: draw the token values on the device (N(0, 1) from a seeded torch
        generator, rounded to bf16) instead of uploading the trace's own values."""
        torch = _torch()
        self.trace = trace
        self.steps = schedule_trace(trace, policy, budget, max_running, num_blocks)
        B = pic.BLOCK_SIZE
        tdt = torch.bfloat16
        if device_seed is None:
            q_all = to_torch(trace.q, "bf16", dev)
            k_all = to_torch(trace.k, "bf16", dev)
            v_all = to_torch(trace.v, "bf16", dev)
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(int(device_seed))
            n = trace.n_tokens
            k_all, v_all, q_all = [torch.randn((n, h, trace.d), generator=g, device=dev).to(tdt)
                                   for h in (trace.hkv, trace.hkv, trace.hq)]
        self.k_pool = torch.full((num_blocks, trace.hkv, B, trace.d), float("nan"), dtype=tdt,
                                 device=dev)
        self.v_pool = torch.full((num_blocks, trace.hkv, trace.d, B), float("nan"), dtype=tdt,
                                 device=dev)
        max_pos = max(trace.composed_len(r) for r in range(len(trace.requests)))
        max_pos = max([max_pos] + list(trace.span_lens))
        self.cos = torch.empty((max_pos, trace.d // 2), dtype=torch.float32, device=dev)
        self.sin = torch.empty_like(self.cos)
        pic.pic_rope_table(self.cos, self.sin, trace.base)
        self.dev_steps = []
        ws = 16
        for st in self.steps:
            if st["num_seqs"] == 0:
                continue
            src = torch.from_numpy(st["src"]).to(dev)
            decode_only = bool(st["max_q_len"] == 1)
            if decode_only:  # one token per sequence, each at its sequence's last key slot
                L = np.asarray(st["seq_lens"], np.int64)
                bt = np.asarray(st["block_table"], np.int64)
                last = bt[np.arange(L.shape[0]), (L - 1) // B] * B + (L - 1) % B
                assert np.array_equal(last, np.asarray(st["slot_mapping"], np.int64))
            d = dict(q=q_all[src].contiguous(), k=k_all[src].contiguous(),
                     v=v_all[src].contiguous(), slots=i32(st["slot_mapping"], dev),
                     cu_q=i32(st["cu_seqlens_q"], dev), q_pos=i32(st["q_pos"], dev),
                     bt=i32(st["block_table"], dev), seq_lens=i32(st["seq_lens"], dev),
                     cu_k=i32(st["cu_seqlens_k"], dev), k_pos=i32(st["k_pos"], dev),
                     max_q_len=st["max_q_len"], max_seq_len=st["max_seq_len"], src=src,
                     decode_only=decode_only)
            d["out"] = torch.empty_like(d["q"])
            ws = max(ws, pic.pic_attn_workspace_size(st["num_seqs"], st["total_q"],
                                                     st["max_seq_len"], trace.hq, trace.hkv,
                                                     trace.d, tdt))
            self.dev_steps.append(d)
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=dev)
        self.rows = int(sum(st["total_q"] for st in self.steps))

    def run(self):
        """Every step: the new tokens' cache write and one attention call.  A step whose
        sequences are all single rows is one decode launch that writes its tokens itself
        (pic_attn_decode_append); any other step is pic_cache_write, then the mixed launch."""
        for d in self.dev_steps:
            if d["decode_only"]:
                pic.pic_attn_decode_append(d["q"], d["k"], d["v"], d["q_pos"], self.k_pool,
                                           self.v_pool, d["bt"], d["seq_lens"], d["cu_k"],
                                           d["k_pos"], self.cos, self.sin, d["max_seq_len"],
                                           d["out"], self.workspace)
            else:
                pic.pic_cache_write(d["k"], d["v"], d["slots"], self.k_pool, self.v_pool)
                pic.pic_attn_prefill(d["q"], d["cu_q"], d["q_pos"], self.k_pool, self.v_pool,
                                     d["bt"], d["seq_lens"], d["cu_k"], d["k_pos"], self.cos,
                                     self.sin, d["max_q_len"], d["max_seq_len"], d["out"],
                                     self.workspace)

    def outputs(self):
        """[n_tokens][Hq][d] float64: each token's output row from its (last) computation,
        and a bool mask of the tokens computed as a one-row sequence (split-KV path)."""
        torch = _torch()
        t = self.trace
        out = torch.full((t.n_tokens, t.hq, t.d), float("nan"), dtype=torch.bfloat16,
                         device=self.k_pool.device)
        single = np.zeros(t.n_tokens, bool)
        for st, d in zip([s for s in self.steps if s["num_seqs"]], self.dev_steps):
            out[d["src"]] = d["out"]
            ql = np.diff(st["cu_seqlens_q"])
            single[st["src"]] = np.repeat(ql == 1, ql)
        return to_f64(out), single

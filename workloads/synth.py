"""Seeded synthetic workloads for position-free paged attention.

Stand-ins for the page's serving workload (MiniPIC §4: 2WikiMultihopQA on a
Llama-3-8B-architecture model, neither of which is present): the layer shape
of Llama-3-8B (32 query heads, 8 kv heads, head size 128) and spans of cached
tokens that several requests reuse at different logical offsets (MiniPIC §1
and §2.1).  Values are N(0, 1); nothing here is model data.

Recipe (the same for every config):

* data RNG ``numpy.random.default_rng(data_seed)`` draws float32
  ``standard_normal`` values in a fixed order: the context tokens' K then V,
  segment by segment, then the step's new tokens' K then V, then the queries;
  bf16 configs round them to nearest-even bfloat16 (kept as uint16 bits);
* structure RNG ``default_rng(100 + data_seed)`` chooses which spans each
  request uses and in which order, and the physical block ids: every logical
  block of the pool gets a physical id from one random permutation, so
  logical and physical order differ;
* logical positions run contiguously over each request's slots in
  composition order (so a shared span sits at a different offset in each
  request that uses it); a decode query sits at the position right after its
  context, and its own new key/value is the request's last slot.

A "step" is what a serving engine does per batch: write the step's new
(unrotated) K/V into the cache, then one attention call.  The context tokens
are resident before the step.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape[0], np.uint16)
    step = 1 << 20                       # chunked: keeps the temporaries in cache
    tmp = np.empty(min(step, flat.shape[0]), np.uint32)
    for a in range(0, flat.shape[0], step):
        u = flat[a:a + step]
        t = tmp[:u.shape[0]]
        np.right_shift(u, 16, out=t)
        np.bitwise_and(t, 1, out=t)
        np.add(t, 0x7FFF, out=t)
        np.add(t, u, out=t)
        np.right_shift(t, 16, out=t)
        out[a:a + step] = t
        nan = np.isnan(u.view(np.float32))
        if nan.any():
            out[a:a + step][nan] = 0x7FC0
    return out.reshape(x.shape)


@dataclasses.dataclass
class Workload:
    name: str
    kind: str            # "decode": every request has one query (pic_attn_decode)
    dtype: str           # "bf16" or "f32" storage / compute type of q, K, V, out
    hq: int
    hkv: int
    d: int
    block_size: int
    base: float
    num_blocks: int
    max_pos: int
    ctx_k: np.ndarray    # [Tc][Hkv][d] resident context tokens (stored values)
    ctx_v: np.ndarray
    ctx_slots: np.ndarray  # [Tc] int32 physical cache slots
    new_k: np.ndarray    # [Tn][Hkv][d] tokens the step writes
    new_v: np.ndarray
    new_slots: np.ndarray  # [Tn] int32
    q: np.ndarray        # [Tq][Hq][d] unrotated queries (stored values)
    cu_seqlens_q: np.ndarray  # [R+1] int32
    q_pos: np.ndarray    # [Tq] int32
    block_table: np.ndarray   # [R][max_blocks] int32 (padding entries are 0)
    seq_lens: np.ndarray      # [R] int32
    cu_seqlens_k: np.ndarray  # [R+1] int32
    k_pos: np.ndarray         # [sum seq_lens] int32, pi(j) per request
    description: str = ""

    @property
    def num_reqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_q_len(self) -> int:
        return int(np.diff(self.cu_seqlens_q).max()) if self.num_reqs else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_reqs else 0

    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q)


# ---------------------------------------------------------------------------
# builder
# ---------------------------------------------------------------------------

_VALUES = [True]


def _draw(rng, shape, dtype):
    """N(0, 1) float32 values drawn in row order, stored as bf16 bits or float32.

    With value drawing switched off (metadata-only builds) it returns a
    read-only zero view of the right shape and draws nothing; the structure
    RNG is separate, so block tables and positions are unchanged.
    """
    if not _VALUES[0]:
        return np.broadcast_to(np.zeros((), np.uint16 if dtype == "bf16" else np.float32), shape)
    if dtype != "bf16":
        return rng.standard_normal(shape, dtype=np.float32)
    out = np.empty(shape, np.uint16)
    rows = out.reshape(shape[0], -1)
    per = max(1, (1 << 20) // max(1, rows.shape[1]))
    for a in range(0, shape[0], per):
        n = min(per, shape[0] - a)
        rows[a:a + n] = f32_to_bf16_bits(rng.standard_normal((n, rows.shape[1]), dtype=np.float32))
    return out


class _Pool:
    """Allocates logical blocks and draws the values of the tokens stored in them."""

    def __init__(self, hkv, d, B, dtype, data_rng):
        self.hkv, self.d, self.B, self.dtype = hkv, d, B, dtype
        self.rng = data_rng
        self.nblocks = 0
        self.k, self.v, self.lslots = [], [], []

    def _draw(self, n):
        return _draw(self.rng, (n, self.hkv, self.d), self.dtype)

    def segment(self, n_tokens):
        """A run of context tokens in fresh blocks; returns its logical block ids."""
        nb = -(-n_tokens // self.B)
        blocks = list(range(self.nblocks, self.nblocks + nb))
        self.nblocks += nb
        self.k.append(self._draw(n_tokens))
        self.v.append(self._draw(n_tokens))
        self.lslots.append(np.asarray(blocks, np.int64)[np.arange(n_tokens) // self.B] * self.B
                           + np.arange(n_tokens) % self.B)
        return blocks

    def empty_blocks(self, nb):
        blocks = list(range(self.nblocks, self.nblocks + nb))
        self.nblocks += nb
        return blocks


def _finish(name, kind, dtype, hq, hkv, d, B, base, pool: _Pool, struct_rng, data_rng,
            requests, new_tokens, q_rows, description):
    """Assemble a Workload.

    requests: list of dicts {blocks: [logical ids], seq_len, k_pos: array}
    new_tokens: list of (request index, slot index within request) written by the step
    q_rows: list of (request index, position) in query-row order, grouped by request
    """
    perm = struct_rng.permutation(pool.nblocks).astype(np.int64)   # logical -> physical

    def phys_slot(lslot):
        lslot = np.asarray(lslot, np.int64)
        return perm[lslot // B] * B + lslot % B

    sdt = np.uint16 if dtype == "bf16" else np.float32
    if pool.k and not _VALUES[0]:
        n_ctx = sum(a.shape[0] for a in pool.k)
        ctx_k = ctx_v = np.broadcast_to(np.zeros((), sdt), (n_ctx, hkv, d))
        ctx_slots = phys_slot(np.concatenate(pool.lslots)).astype(np.int32)
    elif pool.k:
        ctx_k, ctx_v = np.concatenate(pool.k), np.concatenate(pool.v)
        ctx_slots = phys_slot(np.concatenate(pool.lslots)).astype(np.int32)
    else:
        ctx_k = ctx_v = np.zeros((0, hkv, d), sdt)
        ctx_slots = np.zeros(0, np.int32)

    R = len(requests)
    max_blocks = max(len(r["blocks"]) for r in requests)
    block_table = np.zeros((R, max_blocks), np.int32)
    for i, r in enumerate(requests):
        block_table[i, :len(r["blocks"])] = perm[np.asarray(r["blocks"], np.int64)]
    seq_lens = np.array([r["seq_len"] for r in requests], np.int32)
    cu_k = np.zeros(R + 1, np.int32)
    cu_k[1:] = np.cumsum(seq_lens)
    k_pos = np.concatenate([np.asarray(r["k_pos"], np.int64) for r in requests]).astype(np.int32)

    # the step's new tokens
    nslots = []
    for (ri, j) in new_tokens:
        lb = requests[ri]["blocks"][j // B]
        nslots.append(perm[lb] * B + j % B)
    n_new = len(new_tokens)
    new_k = pool._draw(n_new)
    new_v = pool._draw(n_new)
    new_slots = np.asarray(nslots, np.int64).astype(np.int32)

    q = _draw(data_rng, (len(q_rows), hq, d), dtype)
    counts = np.bincount([ri for ri, _ in q_rows], minlength=R)
    cu_q = np.zeros(R + 1, np.int32)
    cu_q[1:] = np.cumsum(counts)
    q_pos = np.array([p for _, p in q_rows], np.int32)
    max_pos = int(max(k_pos.max(), q_pos.max())) + 1
    return Workload(name=name, kind=kind, dtype=dtype, hq=hq, hkv=hkv, d=d, block_size=B,
                    base=base, num_blocks=pool.nblocks, max_pos=max_pos,
                    ctx_k=ctx_k, ctx_v=ctx_v, ctx_slots=ctx_slots,
                    new_k=new_k, new_v=new_v, new_slots=new_slots,
                    q=q, cu_seqlens_q=cu_q, q_pos=q_pos, block_table=block_table,
                    seq_lens=seq_lens, cu_seqlens_k=cu_k, k_pos=k_pos,
                    description=description)


# ---------------------------------------------------------------------------
# configs
# ---------------------------------------------------------------------------

def _tiny(variant: str, seed: int = 1):
    """4 q heads = 4 kv heads, d 64, base 1e4, fp32, block 16.

    One 64-token span stored once in 4 blocks, reused by request A at logical
    offset 0 and request B at offset 2048; each request has 16 suffix tokens
    in a private block, which are also its 16 causal queries (q_len 16,
    seq_len 80).  variant "a": A's and B's suffix q/K/V are identical (so the
    two requests' outputs must agree: only relative positions matter);
    "b": distinct.  variant "d": the 32 suffix queries of "a" replayed as 32
    decode requests with seq_len 65..80.
    """
    hq = hkv = 4
    d, B, base = 64, 16, 10000.0
    data = np.random.default_rng(seed)
    struct = np.random.default_rng(100 + seed)
    pool = _Pool(hkv, d, B, "f32", data)
    span = pool.segment(64)
    suffix_a = pool.empty_blocks(1)
    suffix_b = pool.empty_blocks(1)
    pool.empty_blocks(2)     # spare blocks, so the physical permutation has room
    offs = [0, 2048]
    reqs = []
    for off, sfx in zip(offs, [suffix_a, suffix_b]):
        reqs.append(dict(blocks=span + sfx, seq_len=80, k_pos=np.arange(80) + off))
    # suffix tokens: written by the step at slots 64..79 of each request
    nk = data.standard_normal((16, hkv, d), dtype=np.float32)
    nv = data.standard_normal((16, hkv, d), dtype=np.float32)
    qs = data.standard_normal((16, hq, d), dtype=np.float32)
    if variant == "b":
        nk = np.concatenate([nk, data.standard_normal((16, hkv, d), dtype=np.float32)])
        nv = np.concatenate([nv, data.standard_normal((16, hkv, d), dtype=np.float32)])
        qs = np.concatenate([qs, data.standard_normal((16, hq, d), dtype=np.float32)])
    else:
        nk, nv, qs = np.concatenate([nk, nk]), np.concatenate([nv, nv]), np.concatenate([qs, qs])
    perm = struct.permutation(pool.nblocks).astype(np.int64)

    def pslot(lb, j):
        return int(perm[lb] * B + j % B)

    new_slots = [pslot(reqs[r]["blocks"][(64 + i) // B], 64 + i) for r in range(2) for i in range(16)]
    ctx_slots = (perm[np.asarray(span)[np.arange(64) // B]] * B + np.arange(64) % B).astype(np.int32)
    if variant == "d":
        requests = []
        q_rows_pos = []
        for r in range(2):
            for i in range(16):
                requests.append(dict(blocks=reqs[r]["blocks"], seq_len=65 + i,
                                     k_pos=np.arange(65 + i) + offs[r]))
                q_rows_pos.append(offs[r] + 64 + i)
        kind = "decode"
        cu_q = np.arange(33, dtype=np.int32)
    else:
        requests = reqs
        q_rows_pos = [offs[r] + 64 + i for r in range(2) for i in range(16)]
        kind = "prefill"
        cu_q = np.array([0, 16, 32], np.int32)
    R = len(requests)
    block_table = np.zeros((R, 5), np.int32)
    for i, r in enumerate(requests):
        block_table[i] = perm[np.asarray(r["blocks"], np.int64)]
    seq_lens = np.array([r["seq_len"] for r in requests], np.int32)
    cu_k = np.zeros(R + 1, np.int32)
    cu_k[1:] = np.cumsum(seq_lens)
    k_pos = np.concatenate([r["k_pos"] for r in requests]).astype(np.int32)
    return Workload(
        name="c1" + variant, kind=kind, dtype="f32", hq=hq, hkv=hkv, d=d, block_size=B,
        base=base, num_blocks=pool.nblocks, max_pos=2048 + 80,
        ctx_k=pool.k[0], ctx_v=pool.v[0], ctx_slots=ctx_slots,
        new_k=nk, new_v=nv, new_slots=np.asarray(new_slots, np.int32),
        q=qs, cu_seqlens_q=cu_q, q_pos=np.asarray(q_rows_pos, np.int32),
        block_table=block_table, seq_lens=seq_lens, cu_seqlens_k=cu_k, k_pos=k_pos,
        description=_tiny.__doc__.strip().splitlines()[0])


def _assign_spans(struct, n_req, uses_per_req, n_spans, uses_per_span):
    """Each request gets ``uses_per_req`` distinct spans; each span used ``uses_per_span`` times."""
    assert n_req * uses_per_req == n_spans * uses_per_span
    while True:
        bag = struct.permutation(np.repeat(np.arange(n_spans), uses_per_span))
        rows = bag.reshape(n_req, uses_per_req)
        if all(len(set(r)) == uses_per_req for r in rows):
            return rows


def _decode(name, seed, R, seg_len, n_seg, n_shared, n_spans, hq=32, hkv=8, d=128, B=16,
            base=500000.0, description="", dtype="bf16"):
    """Decode batch: contexts of n_seg segments (n_shared of them shared spans) + new token."""
    # spans are padded to block boundaries (MiniPIC §2.2, Padding primitive)
    assert seg_len % B == 0, "composed segments must fill whole blocks"
    data = np.random.default_rng(seed)
    struct = np.random.default_rng(100 + seed)
    pool = _Pool(hkv, d, B, dtype, data)
    spans = [pool.segment(seg_len) for _ in range(n_spans)]
    uses = (R * n_shared) // n_spans if n_spans else 0
    assign = _assign_spans(struct, R, n_shared, n_spans, uses) if n_shared else None
    requests = []
    for r in range(R):
        shared_slots = set(struct.choice(n_seg, size=n_shared, replace=False).tolist()) if n_shared else set()
        blocks = []
        k = 0
        for s in range(n_seg):
            if s in shared_slots:
                blocks += spans[int(assign[r][k])]
                k += 1
            else:
                blocks += pool.segment(seg_len)
        blocks += pool.empty_blocks(1)          # tail block for the step's new token
        L = n_seg * seg_len + 1
        requests.append(dict(blocks=blocks, seq_len=L, k_pos=np.arange(L)))
    new_tokens = [(r, n_seg * seg_len) for r in range(R)]
    q_rows = [(r, n_seg * seg_len) for r in range(R)]
    return _finish(name, "decode", dtype, hq, hkv, d, B, base, pool, struct, data,
                   requests, new_tokens, q_rows, description)


def _chunked_prefill(seed=3, R=8, n_spans=16, span_len=1024, per_req=4, q_len=512,
                     hq=32, hkv=8, d=128, B=16, base=500000.0, dtype="bf16"):
    """8 requests x (4 distinct seeded spans of 1024 in seeded order + 512 causal suffix queries)."""
    assert span_len % B == 0, "composed spans must fill whole blocks"
    data = np.random.default_rng(seed)
    struct = np.random.default_rng(100 + seed)
    pool = _Pool(hkv, d, B, dtype, data)
    spans = [pool.segment(span_len) for _ in range(n_spans)]
    requests, new_tokens, q_rows = [], [], []
    for r in range(R):
        order = struct.choice(n_spans, size=per_req, replace=False)
        blocks = [b for s in order for b in spans[int(s)]]
        blocks += pool.empty_blocks(-(-q_len // B))
        ctx = per_req * span_len
        L = ctx + q_len
        requests.append(dict(blocks=blocks, seq_len=L, k_pos=np.arange(L)))
        new_tokens += [(r, ctx + i) for i in range(q_len)]
        q_rows += [(r, ctx + i) for i in range(q_len)]
    return _finish("c3", "prefill", dtype, hq, hkv, d, B, base, pool, struct, data,
                   requests, new_tokens, q_rows, _chunked_prefill.__doc__.strip())


def _long_decode(seed=4, R=4, n_spans=64, span_len=2048, hq=32, hkv=8, d=128, B=16,
                 base=500000.0):
    """4 requests x 131072-token contexts: all 64 shared 2048-token spans, each in its own order."""
    data = np.random.default_rng(seed)
    struct = np.random.default_rng(100 + seed)
    pool = _Pool(hkv, d, B, "bf16", data)
    spans = [pool.segment(span_len) for _ in range(n_spans)]
    requests = []
    for r in range(R):
        order = struct.permutation(n_spans)
        blocks = [b for s in order for b in spans[int(s)]]
        blocks += pool.empty_blocks(1)
        L = n_spans * span_len + 1
        requests.append(dict(blocks=blocks, seq_len=L, k_pos=np.arange(L)))
    ctx = n_spans * span_len
    return _finish("c4", "decode", "bf16", hq, hkv, d, B, base, pool, struct, data,
                   requests, [(r, ctx) for r in range(R)], [(r, ctx) for r in range(R)],
                   _long_decode.__doc__.strip())


def _mixed(seed=5, n_chunks=16, chunk=2048, n_dec=128, per_dec=4, hq=32, hkv=8, d=128, B=16,
           base=500000.0, dtype="bf16"):
    """One launch: 16 span-prefill chunks of 2048 (causal within the span) + 128 decodes of
    8192-token contexts built from 4 of those spans each; request order is shuffled."""
    assert chunk % B == 0, "composed spans must fill whole blocks"
    data = np.random.default_rng(seed)
    struct = np.random.default_rng(100 + seed)
    pool = _Pool(hkv, d, B, dtype, data)
    span_blocks = [pool.empty_blocks(chunk // B) for _ in range(n_chunks)]
    reqs = []
    for c in range(n_chunks):
        reqs.append(("prefill", dict(blocks=span_blocks[c], seq_len=chunk, k_pos=np.arange(chunk)), c))
    for r in range(n_dec):
        order = struct.choice(n_chunks, size=per_dec, replace=False)
        blocks = [b for s in order for b in span_blocks[int(s)]]
        blocks += pool.empty_blocks(1)
        L = per_dec * chunk + 1
        reqs.append(("decode", dict(blocks=blocks, seq_len=L, k_pos=np.arange(L)), r))
    order = struct.permutation(len(reqs))
    requests, new_tokens, q_rows = [], [], []
    for idx, o in enumerate(order):
        kind, rq, _ = reqs[int(o)]
        requests.append(rq)
        if kind == "prefill":
            new_tokens += [(idx, j) for j in range(chunk)]
            q_rows += [(idx, j) for j in range(chunk)]
        else:
            new_tokens.append((idx, per_dec * chunk))
            q_rows.append((idx, per_dec * chunk))
    return _finish("c5", "prefill", dtype, hq, hkv, d, B, base, pool, struct, data,
                   requests, new_tokens, q_rows, _mixed.__doc__.strip().replace("\n    ", " "))


CONFIGS = {
    "c1a": lambda: _tiny("a"),
    "c1b": lambda: _tiny("b"),
    "c1d": lambda: _tiny("d"),
    "c2": lambda: _decode("c2", 2, R=64, seg_len=1024, n_seg=4, n_shared=2, n_spans=32,
                          description="decode: 64 requests x 4096-token context (2 of 4 "
                          "1024-token segments are shared spans) + 1 new token each"),
    "c2p": lambda: _decode("c2p", 2, R=64, seg_len=1024, n_seg=4, n_shared=0, n_spans=0,
                           description="decode, private control: same shape, no sharing"),
    "c3": _chunked_prefill,
    "c4": _long_decode,
    "c5": _mixed,
}


def make_workload(name: str, values: bool = True, **overrides) -> Workload:
    """Build a named config (or, with ``builder=...``, a resized variant of one).

    values=False skips drawing K/V/q values (metadata only: same block tables,
    slots and positions, since those come from the separate structure RNG).
    """
    _VALUES[0] = values
    try:
        if overrides:
            builders = {"decode": _decode, "prefill": _chunked_prefill, "long": _long_decode,
                        "mixed": _mixed}
            kind = overrides.pop("builder")
            if kind == "decode":
                overrides["name"] = name
            return builders[kind](**overrides)
        return CONFIGS[name]()
    finally:
        _VALUES[0] = True


# ---------------------------------------------------------------------------
# measurement bookkeeping (counts, not the method's arithmetic)
# ---------------------------------------------------------------------------

def algorithmic_counts(w: Workload) -> dict:
    """Bytes and flops one attention call must move / do.

    bytes: K and V of every (request, visible key slot, kv head) counted per
    request (each request attends to its whole context even where blocks are
    shared), plus q, out, block-table entries used, k_pos, q_pos, seq_lens /
    cu_seqlens, and one cos/sin row (d/2 fp32 each) per distinct position
    used.  unique_kv_bytes counts each physical block once.
    flops: 4 d per unmasked (query row, key slot, q head) -- QK^T and PV.
    """
    es = 2 if w.dtype == "bf16" else 4
    ql = w.q_lens().astype(np.int64)
    L = w.seq_lens.astype(np.int64)
    kv_row = w.hkv * w.d * es * 2
    kv = int((L * kv_row).sum())
    # visible (row, key) pairs: row i of q_len sees L - q_len + i + 1 slots
    pairs = int(sum(int(ql_r * (Lr - ql_r) + ql_r * (ql_r + 1) // 2) for ql_r, Lr in zip(ql, L)))
    q_out = 2 * w.total_q * w.hq * w.d * es
    blocks_used = int(sum(-(-int(x) // w.block_size) for x in L))
    meta = 4 * (blocks_used + int(L.sum()) + w.total_q + 2 * w.num_reqs + 1)
    positions = np.unique(np.concatenate([w.k_pos, w.q_pos]))
    table = int(positions.shape[0]) * (w.d // 2) * 4 * 2
    touched = np.unique(np.concatenate([w.block_table[r, :-(-int(L[r]) // w.block_size)]
                                        for r in range(w.num_reqs)]))
    unique_kv = int(touched.shape[0]) * w.block_size * kv_row
    return dict(bytes=kv + q_out + meta + table, kv_bytes=kv, unique_kv_bytes=unique_kv,
                table_bytes=table, flops=4 * w.d * w.hq * pairs, score_pairs=pairs * w.hq)

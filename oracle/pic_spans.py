"""Reference for span-aware block hashing (TEST INFRASTRUCTURE ONLY).

Follows "MiniPIC: Flexible Position-Independent Caching in <100LOC", §2.2
(user-controlled cache-reuse primitives):

* Padding: spans are padded to KV-block boundaries so that the special
  tokens sit at the start of a block (the caller's job; nothing to compute);
* SSEP at the start of a block restarts the hash chain, h_i = H(h_0, x_i),
  so a span hashes the same whatever context precedes it;
* PDEP at the start of a block makes the hash depend on the whole preceding
  prompt, h_i = H(h_0, x_<=i), so a suffix block that depends on its context
  never matches a block computed under another context.

Readings where the page is silent: a block without a special token chains on
its predecessor, h_i = H(h_{i-1}, x_i) with h_{-1} = h_0 (the usual prefix
cache; the page's two formulas only make sense against it); x_<=i means
every token of blocks 0..i of the prompt; only full blocks are hashed.
H(parent, tokens) is FNV-1a 64 (Fowler, Noll, Vo) of the byte string
parent as 8 little-endian bytes followed by each token id as 4 little-endian
bytes (two's complement).  This module builds those byte strings explicitly
and hashes them from scratch, with no running state.
"""

from __future__ import annotations

import struct

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit: for each byte, xor it in, then multiply by the prime (mod 2^64)."""
    h = FNV_OFFSET
    for b in data:
        h = ((h ^ b) * FNV_PRIME) & MASK64
    return h


def _h(parent: int, tokens) -> int:
    data = struct.pack("<Q", parent) + b"".join(struct.pack("<i", int(t)) for t in tokens)
    return fnv1a64(data)


def block_hashes(tokens, block_size: int, ssep: int = -1, pdep: int = -1, seed: int = 0):
    """Hashes of the full blocks of one prompt, by the three rules above."""
    tokens = [int(t) for t in tokens]
    out = []
    parent = seed
    for i in range(len(tokens) // block_size):
        x = tokens[i * block_size:(i + 1) * block_size]
        if pdep >= 0 and x[0] == pdep:
            h = _h(seed, tokens[:(i + 1) * block_size])
        elif ssep >= 0 and x[0] == ssep:
            h = _h(seed, x)
        else:
            h = _h(parent, x)
        out.append(h)
        parent = h
    return out


def build_block_tables(prompts, block_size: int, ssep: int = -1, pdep: int = -1, seed: int = 0,
                       first_block: int = 0):
    """Block table rows, positions and slot mappings of a batch of prompts.

    Full blocks with equal hashes share one physical block, numbered in order of
    first use; a partial last block is always private.  Positions are the token
    indices 0..len-1 of each prompt.  A token whose block was already written by
    an earlier occurrence gets slot -1.
    """
    owner = {}
    nxt = first_block
    tables, k_pos, slots = [], [], []
    for toks in prompts:
        n = len(toks)
        hs = block_hashes(toks, block_size, ssep, pdep, seed)
        row, sl = [], []
        for b in range(-(-n // block_size)):
            fresh = True
            if b < len(hs):
                if hs[b] in owner:
                    blk, fresh = owner[hs[b]], False
                else:
                    blk = owner[hs[b]] = nxt
                    nxt += 1
            else:
                blk = nxt
                nxt += 1
            row.append(blk)
            for j in range(min(block_size, n - b * block_size)):
                sl.append(blk * block_size + j if fresh else -1)
        tables.append(row)
        k_pos.append(list(range(n)))
        slots.append(sl)
    return tables, k_pos, slots, nxt - first_block

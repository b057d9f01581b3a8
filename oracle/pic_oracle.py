"""fp64 reference for position-free paged attention (TEST INFRASTRUCTURE ONLY).

Follows "MiniPIC: Flexible Position-Independent Caching in <100LOC", §2.1
(Position-free KV implementation):

* the cache holds unrotated key vectors k~_j (§2.1, first paragraph);
* score(t, j) = (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d), with R a rotation
  matrix and pi(j) the logical position of stored key j in the current
  request (§2.1, score equation);
* one physical block may be referenced by several requests at different
  offsets (§2.1, "Advantage" bullet), so each request brings its own pi;
* applying the rotation inside attention is algebraically the same as
  re-rotating the cache hit (§2.1, "Implementation" bullet) -- i.e. the result
  is plain softmax attention over keys rotated to their logical positions,
  which is exactly what this module computes, densely and without any online
  softmax, blocking or fusion.

Readings where the page is silent:

* R_p is the rotate-half RoPE rotation: element i is paired with element
  i + d/2 and the pair is rotated by angle p * theta_i, with the standard
  frequencies theta_i = base^(-2i/d), i in [0, d/2).
* V is not rotated (the page rotates only keys and queries).
* The query of row i (0-based) of a request with q_len query rows and
  seq_len key slots sees slots j <= seq_len - q_len + i (causal mask aligned
  to the bottom right, over slot index, never over position).
* Grouped-query attention: q head h reads kv head h // (Hq / Hkv).
* Softmax uses the natural exponential; scale 1/sqrt(d) as in the equation.

Storage layout (the boundary's own choice, documented in include/pic.h):
k_pool[num_blocks][Hkv][B][d] and v_pool[num_blocks][Hkv][d][B] (V is stored
transposed inside each block).  Slot s of the cache is block s // B, offset
s % B.  The pools hold the stored values: float32, or bfloat16 kept as uint16
bit patterns.  Everything is upcast exactly to float64 before any arithmetic.
"""

from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# value domain
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns (uint16) to float64.

    A bfloat16 is the top 16 bits of an IEEE float32, so shifting the pattern
    into the high half of a 32-bit word gives the identical float32 value.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _to_f64(stored: np.ndarray) -> np.ndarray:
    if stored.dtype == np.uint16:
        return bf16_bits_to_f64(stored)
    if stored.dtype == np.float32 or stored.dtype == np.float64:
        return stored.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {stored.dtype}")


# ---------------------------------------------------------------------------
# rotation (MiniPIC §2.1: R is the rotation matrix of rotary position embedding)
# ---------------------------------------------------------------------------

def rope_frequencies(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d) for i in [0, d/2), in float64 (standard RoPE)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / head_dim)


def rope_table(max_pos: int, head_dim: int, base: float):
    """cos/sin lookup table [max_pos][d/2]: cos(p * theta_i), sin(p * theta_i).

    This is the "cosine/sine table" the attention kernel looks up for every
    key element (MiniPIC §2.1, Implementation bullet).  Angles and the trig
    functions are evaluated in float64.
    """
    theta = rope_frequencies(head_dim, base)
    p = np.arange(max_pos, dtype=np.float64)
    ang = p[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def rotate_half(x: np.ndarray, pos, head_dim: int, base: float) -> np.ndarray:
    """Apply R_pos to vectors x[..., d] (rotate-half pairing), float64.

    For pair index i in [0, d/2) with angle a = pos * theta_i:
        y_i       = x_i cos a - x_{i+d/2} sin a
        y_{i+d/2} = x_{i+d/2} cos a + x_i sin a
    ``pos`` broadcasts against x[..., 0].
    """
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] != head_dim:
        raise ValueError("last axis must be head_dim")
    h = head_dim // 2
    theta = rope_frequencies(head_dim, base)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ---------------------------------------------------------------------------
# paged storage (MiniPIC §2.1: unrotated keys in shared physical blocks)
# ---------------------------------------------------------------------------

def place_tokens(k_tok, v_tok, slot_mapping, k_pool, v_pool, block_size: int):
    """Store unrotated K~/V of tokens into the pools, in place.

    k_tok, v_tok: [T][Hkv][d] stored values; slot_mapping[T]: cache slot of
    each token (block * B + offset); a negative slot means "skip this token".
    No arithmetic: the stored bits are copied.
    """
    slot_mapping = np.asarray(slot_mapping)
    for t in range(slot_mapping.shape[0]):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        b, o = divmod(s, block_size)
        k_pool[b, :, o, :] = k_tok[t]
        v_pool[b, :, :, o] = v_tok[t]


def gather_request(k_pool, v_pool, block_table_row, seq_len: int, block_size: int):
    """Key slots 0..seq_len-1 of one request, as stored: K~[L][Hkv][d], V[L][Hkv][d]."""
    hkv, d = k_pool.shape[1], k_pool.shape[3]
    kt = np.empty((seq_len, hkv, d), dtype=k_pool.dtype)
    vt = np.empty((seq_len, hkv, d), dtype=v_pool.dtype)
    for j in range(seq_len):
        phys = int(block_table_row[j // block_size])
        off = j % block_size
        kt[j] = k_pool[phys, :, off, :]
        vt[j] = v_pool[phys, :, :, off]
    return kt, vt


# ---------------------------------------------------------------------------
# attention (MiniPIC §2.1 score equation + ordinary softmax attention)
# ---------------------------------------------------------------------------

def attention_request(q, q_pos, k_unrot, v, k_pos, q_len: int, base: float,
                      num_kv_heads: int, rows=None):
    """Outputs of one request, float64.

    q: [q_len][Hq][d] stored (unrotated) queries; q_pos[q_len] their logical
    positions t; k_unrot/v: [L][Hkv][d] stored keys/values of the request's
    key slots in slot order; k_pos[L] = pi(j).  ``rows`` optionally selects
    query rows (indices into q_len); returns [len(rows)][Hq][d].
    """
    q = _to_f64(np.asarray(q))
    k_unrot = _to_f64(np.asarray(k_unrot))
    v = _to_f64(np.asarray(v))
    L = k_unrot.shape[0]
    hq, d = q.shape[1], q.shape[2]
    group = hq // num_kv_heads
    if rows is None:
        rows = np.arange(q_len)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], hq, d), dtype=np.float64)
    if rows.shape[0] == 0:
        return out
    # keys rotated to their logical positions pi(j) in this request
    k_rot = rotate_half(k_unrot, np.asarray(k_pos)[:, None], d, base)  # [L][Hkv][d]
    q_rot = rotate_half(q[rows], np.asarray(q_pos)[rows][:, None], d, base)  # [n][Hq][d]
    scale = 1.0 / np.sqrt(np.float64(d))
    # number of visible key slots for each selected row
    visible = L - q_len + rows + 1
    for h in range(hq):
        g = h // group
        s = (q_rot[:, h, :] @ k_rot[:, g, :].T) * scale  # [n][L]
        for n in range(rows.shape[0]):
            nv = int(visible[n])
            if nv <= 0:
                continue
            sv = s[n, :nv]
            w = np.exp(sv - sv.max())
            w /= w.sum()
            out[n, h, :] = w @ v[:nv, g, :]
    return out


def attention(q, cu_seqlens_q, q_pos, k_pool, v_pool, block_table, seq_lens,
              cu_seqlens_k, k_pos, base: float, block_size: int, requests=None,
              rows=None):
    """Batched reference: returns {r: [q_len_r or len(rows[r])][Hq][d] float64}.

    q[Tq][Hq][d]; request r owns query rows cu_seqlens_q[r]..cu_seqlens_q[r+1]
    and key slots 0..seq_lens[r]-1, whose logical positions are
    k_pos[cu_seqlens_k[r] : cu_seqlens_k[r] + seq_lens[r]].
    ``requests`` selects requests; ``rows`` maps a request to the query rows
    (within the request) to evaluate.
    """
    hkv = k_pool.shape[1]
    if requests is None:
        requests = range(len(seq_lens))
    res = {}
    for r in requests:
        q0, q1 = int(cu_seqlens_q[r]), int(cu_seqlens_q[r + 1])
        L = int(seq_lens[r])
        kt, vt = gather_request(k_pool, v_pool, block_table[r], L, block_size)
        k0 = int(cu_seqlens_k[r])
        sel = None if rows is None else rows.get(r)
        res[r] = attention_request(q[q0:q1], q_pos[q0:q1], kt, vt,
                                   k_pos[k0:k0 + L], q1 - q0, base, hkv, sel)
    return res

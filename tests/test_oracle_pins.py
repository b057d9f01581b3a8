"""Pins for the fp64 oracle: things it must agree with that are not the oracle.

Each check ties the oracle to something fixed independently of its own code:

* brute force: pure-Python loops with explicit d x d rotation matrices
  (2x2 blocks on the pairs (i, i + d/2)), an independent paged gather, and a
  softmax without max subtraction, on tiny inputs;
* pre-rotated equality: rotating keys with complex multiplication (a second,
  independent formulation of the same rotation), then running the library
  attention routine (torch SDPA in float64) with an explicit bottom-right
  mask -- the page states that in-kernel rotation equals re-rotating the hit
  (MiniPIC §2.1, Implementation bullet);
* shift invariance: rotary scores depend only on position differences
  (R_a^T R_b = R_{b-a}), so shifting every position of a request by c leaves
  scores and outputs unchanged;
* closed forms: a hand-computed rotation, exact frequencies for base 10^4 at
  d = 8, one visible key gives V exactly, zero keys give the mean of V, equal
  scores give the midpoint, rotations are orthogonal;
* mutation checks: plausible mistakes planted into copies of the oracle on the
  CPU (sign, pairing, frequency, GQA map, V layout, mask alignment) must each
  be caught by one of the pins above.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import pic_oracle as po


# ---------------------------------------------------------------------------
# brute force, written independently of oracle/ (loops, explicit matrices)
# ---------------------------------------------------------------------------

def bf_rotation_matrix(p, d, base):
    h = d // 2
    R = [[0.0] * d for _ in range(d)]
    for i in range(h):
        a = p * base ** (-2.0 * i / d)
        c, s = math.cos(a), math.sin(a)
        R[i][i] = c
        R[i][i + h] = -s
        R[i + h][i] = s
        R[i + h][i + h] = c
    return R


def bf_matvec(M, x):
    return [sum(M[r][c] * x[c] for c in range(len(x))) for r in range(len(M))]


def bf_attention(q, q_pos, k_pool, v_pool, block_table, seq_lens, cu_q, cu_k, k_pos,
                 base, B):
    """q[Tq][Hq][d] floats; pools in the documented layouts; returns nested lists."""
    R_ = len(seq_lens)
    hq = len(q[0])
    d = len(q[0][0])
    hkv = len(k_pool[0])
    G = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(len(q))]
    for r in range(R_):
        L = seq_lens[r]
        ql = cu_q[r + 1] - cu_q[r]
        keys, vals = [], []
        for j in range(L):
            blk = block_table[r][j // B]
            off = j % B
            keys.append([[k_pool[blk][g][off][e] for e in range(d)] for g in range(hkv)])
            vals.append([[v_pool[blk][g][e][off] for e in range(d)] for g in range(hkv)])
        for i in range(ql):
            row = cu_q[r] + i
            Rt = bf_rotation_matrix(q_pos[row], d, base)
            nvis = L - ql + i + 1
            for h in range(hq):
                g = h // G
                qr = bf_matvec(Rt, q[row][h])
                sc = []
                for j in range(nvis):
                    Rp = bf_rotation_matrix(k_pos[cu_k[r] + j], d, base)
                    kr = bf_matvec(Rp, keys[j][g])
                    sc.append(sum(qr[e] * kr[e] for e in range(d)) / math.sqrt(d))
                ex = [math.exp(s) for s in sc]
                tot = sum(ex)
                for e in range(d):
                    out[row][h][e] = sum(ex[j] * vals[j][g][e] for j in range(nvis)) / tot
    return out


# ---------------------------------------------------------------------------
# a tiny paged batch with sharing, GQA, repeated / non-monotone positions
# ---------------------------------------------------------------------------

def tiny_batch(seed, d=8, hq=4, hkv=2, B=4, base=10000.0, shift=None):
    rng = np.random.default_rng(seed)
    nb = 7
    k_pool = rng.standard_normal((nb, hkv, B, d))
    v_pool = rng.standard_normal((nb, hkv, d, B))
    # request 0: 3 blocks, 10 slots, 3 queries; request 1 shares block 4 and
    # block 1 at other offsets, 6 slots, 1 query; request 2: 5 slots, 5 queries
    block_table = np.array([[4, 1, 6], [1, 4, 0], [2, 5, 0]], dtype=np.int32)
    seq_lens = [10, 6, 5]
    q_lens = [3, 1, 5]
    cu_q = [0, 3, 4, 9]
    cu_k = [0, 10, 16, 21]
    k_pos = np.concatenate([
        np.arange(100, 110),                 # contiguous at offset 100
        np.array([7, 3, 3, 50, 2, 900]),     # repeated and non-monotone
        np.arange(5),
    ]).astype(np.int64)
    q_pos = np.array([107, 108, 109, 901, 0, 1, 2, 3, 4], dtype=np.int64)
    if shift is not None:
        k_pos = k_pos + shift
        q_pos = q_pos + shift
    q = rng.standard_normal((9, hq, d))
    return dict(q=q, q_pos=q_pos, k_pool=k_pool, v_pool=v_pool, block_table=block_table,
                seq_lens=seq_lens, q_lens=q_lens, cu_q=cu_q, cu_k=cu_k, k_pos=k_pos,
                base=base, B=B, d=d, hq=hq, hkv=hkv)


def run_oracle(b, mod=po):
    res = mod.attention(b["q"], b["cu_q"], b["q_pos"], b["k_pool"], b["v_pool"],
                        b["block_table"], b["seq_lens"], b["cu_k"], b["k_pos"],
                        b["base"], b["B"])
    return np.concatenate([res[r] for r in range(len(b["seq_lens"]))], axis=0)


def run_brute(b):
    return np.array(bf_attention(b["q"].tolist(), b["q_pos"].tolist(), b["k_pool"].tolist(),
                                 b["v_pool"].tolist(), b["block_table"].tolist(), b["seq_lens"],
                                 b["cu_q"], b["cu_k"], b["k_pos"].tolist(), b["base"], b["B"]))


@pytest.mark.parametrize("seed,d,base", [(0, 8, 10000.0), (1, 4, 10000.0), (2, 8, 500000.0)])
def test_brute_force_matches(seed, d, base):
    b = tiny_batch(seed, d=d, base=base)
    np.testing.assert_allclose(run_oracle(b), run_brute(b), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# pre-rotated equality with the library attention routine
# ---------------------------------------------------------------------------

def complex_rotate(x, pos, base):
    """Rotate-half RoPE as complex multiplication: z_i = x_i + i x_{i+d/2}."""
    d = x.shape[-1]
    h = d // 2
    theta = base ** (-np.arange(h) * 2.0 / d)
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def prerotated_sdpa(b):
    """What a rotated cache would hold, then library attention with an explicit mask."""
    outs = []
    G = b["hq"] // b["hkv"]
    for r in range(len(b["seq_lens"])):
        L = b["seq_lens"][r]
        q0, q1 = b["cu_q"][r], b["cu_q"][r + 1]
        ql = q1 - q0
        bt = b["block_table"][r]
        slots = np.arange(L)
        K = b["k_pool"][bt[slots // b["B"]], :, slots % b["B"], :]          # [L][Hkv][d]
        V = b["v_pool"][bt[slots // b["B"]], :, :, slots % b["B"]]          # [L][Hkv][d]
        kp = b["k_pos"][b["cu_k"][r]:b["cu_k"][r] + L]
        Kr = complex_rotate(K, kp[:, None], b["base"])
        Qr = complex_rotate(b["q"][q0:q1], b["q_pos"][q0:q1][:, None], b["base"])
        qt = torch.from_numpy(Qr).permute(1, 0, 2)[None]                     # [1][Hq][ql][d]
        kt = torch.from_numpy(Kr).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        i = torch.arange(ql)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= (L - ql + i)          # bottom-right aligned
        o = F.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(), attn_mask=mask)
        outs.append(o[0].permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)


@pytest.mark.parametrize("seed,base", [(3, 10000.0), (4, 500000.0)])
def test_prerotated_equality(seed, base):
    b = tiny_batch(seed, d=16, base=base)
    np.testing.assert_allclose(run_oracle(b), prerotated_sdpa(b), rtol=0, atol=1e-12)


def test_prerotated_equality_larger():
    """Same check at Llama-3 head size with long positions."""
    rng = np.random.default_rng(5)
    b = tiny_batch(5, d=128, hq=8, hkv=2, B=16, base=500000.0)
    b["k_pool"] = rng.standard_normal((7, 2, 16, 128))
    b["v_pool"] = rng.standard_normal((7, 2, 128, 16))
    b["k_pos"] = rng.integers(0, 131072, size=b["k_pos"].shape[0])
    b["q_pos"] = rng.integers(0, 131072, size=b["q_pos"].shape[0])
    b["q"] = rng.standard_normal((9, 8, 128))
    b["block_table"] = np.array([[4, 1, 6], [1, 4, 0], [2, 5, 0]], dtype=np.int32)
    b["seq_lens"] = [40, 20, 16]
    b["cu_k"] = [0, 40, 60, 76]
    b["k_pos"] = rng.integers(0, 131072, size=76)
    np.testing.assert_allclose(run_oracle(b), prerotated_sdpa(b), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# relative-position property
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("c", [1, 2048, 100000, 7919])
def test_shift_invariance_scores_and_outputs(c):
    d, base = 128, 500000.0
    rng = np.random.default_rng(6)
    q = rng.standard_normal((5, d))
    k = rng.standard_normal((5, d))
    tq = rng.integers(0, 5000, size=5)
    tk = rng.integers(0, 5000, size=5)
    s0 = (po.rotate_half(q, tq, d, base) * po.rotate_half(k, tk, d, base)).sum(-1)
    s1 = (po.rotate_half(q, tq + c, d, base) * po.rotate_half(k, tk + c, d, base)).sum(-1)
    np.testing.assert_allclose(s1, s0, rtol=0, atol=1e-5)
    b0 = tiny_batch(7, d=16, base=base)
    b1 = tiny_batch(7, d=16, base=base, shift=c)
    np.testing.assert_allclose(run_oracle(b1), run_oracle(b0), rtol=0, atol=1e-5)


def test_relative_rotation_identity():
    """<R_a x, R_b y> = <x, R_(b-a) y>."""
    d, base = 64, 10000.0
    rng = np.random.default_rng(8)
    x, y = rng.standard_normal(d), rng.standard_normal(d)
    for a, b_ in [(0, 5), (17, 3), (1000, 4096), (131072, 77)]:
        lhs = po.rotate_half(x, a, d, base) @ po.rotate_half(y, b_, d, base)
        rhs = x @ po.rotate_half(y, b_ - a, d, base)
        assert abs(lhs - rhs) < 1e-9


# ---------------------------------------------------------------------------
# closed forms and special cases
# ---------------------------------------------------------------------------

def test_rotate_half_hand_example():
    base = 10000.0
    t1 = base ** -0.5            # theta_1 at d = 4
    r = po.rotate_half(np.array([1.0, 0, 0, 0]), 1, 4, base)
    np.testing.assert_allclose(r, [math.cos(1), 0, math.sin(1), 0], atol=1e-15)
    r = po.rotate_half(np.array([0, 1.0, 0, 0]), 1, 4, base)
    np.testing.assert_allclose(r, [0, math.cos(t1), 0, math.sin(t1)], atol=1e-15)
    r = po.rotate_half(np.array([0, 0, 1.0, 0]), 1, 4, base)
    np.testing.assert_allclose(r, [-math.sin(1), 0, math.cos(1), 0], atol=1e-15)
    r = po.rotate_half(np.array([0, 0, 0, 1.0]), 2, 4, base)
    np.testing.assert_allclose(r, [0, -math.sin(2 * t1), 0, math.cos(2 * t1)], atol=1e-15)


def test_frequencies_closed_form():
    # base 10^4, d = 8: theta_i = 10^(-i) exactly as decimal powers
    th = po.rope_frequencies(8, 10000.0)
    np.testing.assert_allclose(th, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    # base 5e5, d = 128: theta_0 = 1, theta_63 = 5e5^(-126/128)
    th = po.rope_frequencies(128, 500000.0)
    assert th[0] == 1.0
    assert abs(th[63] - math.exp(-126 / 128 * math.log(500000.0))) < 1e-18


def test_rope_table_values():
    cos_t, sin_t = po.rope_table(5000, 8, 10000.0)
    for p in [0, 1, 2, 77, 4999]:
        for i, th in enumerate([1.0, 0.1, 0.01, 0.001]):
            assert abs(cos_t[p, i] - math.cos(p * th)) < 1e-15
            assert abs(sin_t[p, i] - math.sin(p * th)) < 1e-15
    assert np.all(cos_t[0] == 1.0) and np.all(sin_t[0] == 0.0)


def test_rotation_is_orthogonal():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((50, 128))
    p = rng.integers(0, 131073, size=50)
    y = po.rotate_half(x, p, 128, 500000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-13)


def test_identity_positions_equal_plain_attention():
    b = tiny_batch(10, d=8)
    b["k_pos"] = np.zeros_like(b["k_pos"])
    b["q_pos"] = np.zeros_like(b["q_pos"])
    got = run_oracle(b)
    # plain attention on the unrotated values through the library routine
    ref = prerotated_sdpa(dict(b, base=b["base"]))
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_single_visible_key_returns_v_exactly():
    # q_len == seq_len: the first query row sees slot 0 only
    b = tiny_batch(11, d=8)
    out = run_oracle(b)
    r = 2
    row0 = b["cu_q"][r]
    blk = b["block_table"][r][0]
    for h in range(b["hq"]):
        g = h // (b["hq"] // b["hkv"])
        assert np.array_equal(out[row0, h], b["v_pool"][blk, g, :, 0])


def test_zero_keys_give_mean_of_visible_values():
    b = tiny_batch(12, d=8)
    b["k_pool"] = np.zeros_like(b["k_pool"])
    out = run_oracle(b)
    r = 0
    L, ql = b["seq_lens"][r], b["q_lens"][r]
    slots = np.arange(L)
    V = b["v_pool"][b["block_table"][r][slots // 4], :, :, slots % 4]
    for i in range(ql):
        nv = L - ql + i + 1
        for h in range(b["hq"]):
            g = h // 2
            np.testing.assert_allclose(out[b["cu_q"][r] + i, h], V[:nv, g].mean(0), atol=1e-15)


def test_two_equal_scores_give_midpoint():
    d = 4
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    k_tok = np.array([[1.0, 0, 0, 0], [1.0, 0, 0, 0]])[:, None, :]
    v_tok = np.array([[2.0, 4, 6, 8], [4.0, 0, 2, 0]])[:, None, :]
    out = po.attention_request(q, np.array([3]), k_tok, v_tok, np.array([3, 3]), 1, 10000.0, 1)
    np.testing.assert_allclose(out[0, 0], [3.0, 2.0, 4.0, 4.0], atol=1e-15)


def test_bf16_upcast_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = po.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 0.0
    assert vals[2] == 3.140625
    assert vals[5] == (2 - 2 ** -7) * 2.0 ** 127
    assert vals[6] == 2.0 ** -133


# ---------------------------------------------------------------------------
# storage layout of the pools (the boundary's documented layout)
# ---------------------------------------------------------------------------

def test_place_and_gather_layout():
    rng = np.random.default_rng(13)
    nb, hkv, B, d = 5, 3, 4, 6
    T = 9
    k_tok = rng.integers(0, 65535, size=(T, hkv, d)).astype(np.uint16)
    v_tok = rng.integers(0, 65535, size=(T, hkv, d)).astype(np.uint16)
    slots = np.array([13, 0, 7, -1, 19, 4, 5, 6, -5])
    kp = np.zeros((nb, hkv, B, d), np.uint16)
    vp = np.zeros((nb, hkv, d, B), np.uint16)
    po.place_tokens(k_tok, v_tok, slots, kp, vp, B)
    kflat, vflat = kp.reshape(-1), vp.reshape(-1)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), B)
        for g in range(hkv):
            for e in range(d):
                assert kflat[((blk * hkv + g) * B + off) * d + e] == k_tok[t, g, e]
                assert vflat[((blk * hkv + g) * d + e) * B + off] == v_tok[t, g, e]
    untouched = np.ones(nb * B, bool)
    untouched[slots[slots >= 0]] = False
    for s in np.nonzero(untouched)[0]:
        blk, off = divmod(int(s), B)
        assert not kp[blk, :, off, :].any() and not vp[blk, :, :, off].any()
    # gather through a block table returns tokens in slot order:
    # table [3, 1] -> slots 12..15 then 4..7 -> tokens (-, 0, -, -, 5, 6, 7, 2)
    kt, vt = po.gather_request(kp, vp, np.array([3, 1]), 8, B)
    for j, t in [(1, 0), (4, 5), (5, 6), (6, 7), (7, 2)]:
        assert np.array_equal(kt[j], k_tok[t]) and np.array_equal(vt[j], v_tok[t])


# ---------------------------------------------------------------------------
# mutation checks: planted mistakes in copies of the oracle must be caught
# ---------------------------------------------------------------------------

def _mut_sign(x, pos, d, base):
    h = d // 2
    th = po.rope_frequencies(d, base)
    a = np.asarray(pos, dtype=np.float64)[..., None] * th
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * np.cos(a) + hi * np.sin(a), hi * np.cos(a) - lo * np.sin(a)], -1)


def _mut_interleaved(x, pos, d, base):
    th = po.rope_frequencies(d, base)
    a = np.asarray(pos, dtype=np.float64)[..., None] * th
    ev, od = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = ev * np.cos(a) - od * np.sin(a)
    y[..., 1::2] = od * np.cos(a) + ev * np.sin(a)
    return y


def _mut_freq(x, pos, d, base):
    h = d // 2
    th = np.power(base, -np.arange(h) / d)   # dropped factor 2
    a = np.asarray(pos, dtype=np.float64)[..., None] * th
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * np.cos(a) - hi * np.sin(a), hi * np.cos(a) + lo * np.sin(a)], -1)


_orig_gather = po.gather_request


def _mut_gather_v_transposed(k_pool, v_pool, bt, L, B):
    kt, vt = _orig_gather(k_pool, v_pool, bt, L, B)
    d = k_pool.shape[3]
    for j in range(L):
        vt[j] = v_pool[int(bt[j // B])].reshape(-1, B, d)[:, j % B, :]
    return kt, vt


def _mut_gather_block_offset(k_pool, v_pool, bt, L, B):
    kt, vt = _orig_gather(k_pool, v_pool, bt, L, B)
    for j in range(L):
        kt[j] = k_pool[int(bt[j // B]), :, (j + 1) % B, :]
    return kt, vt


@pytest.mark.parametrize("name,target,mutant", [
    ("sign", "rotate_half", _mut_sign),
    ("interleaved pairing", "rotate_half", _mut_interleaved),
    ("frequency exponent", "rotate_half", _mut_freq),
    ("V read untransposed", "gather_request", _mut_gather_v_transposed),
    ("slot offset", "gather_request", _mut_gather_block_offset),
])
def test_pins_catch_planted_mistakes(monkeypatch, name, target, mutant):
    b = tiny_batch(14, d=8)
    ref = run_brute(b)
    monkeypatch.setattr(po, target, mutant)
    got = run_oracle(b)
    assert np.abs(got - ref).max() > 1e-3, name


def test_pins_catch_mask_and_gqa_mistakes(monkeypatch):
    b = tiny_batch(15, d=8)
    ref = run_brute(b)
    orig = po.attention_request

    def top_left_mask(q, q_pos, k_unrot, v, k_pos, q_len, base, hkv, rows=None):
        # mistake: row i sees slots 0..i (causal limit counted from the top left)
        rows = np.arange(q_len) if rows is None else np.asarray(rows)
        return np.concatenate([orig(q[i:i + 1], q_pos[i:i + 1], k_unrot[:i + 1], v[:i + 1],
                                    k_pos[:i + 1], 1, base, hkv) for i in rows], axis=0)

    monkeypatch.setattr(po, "attention_request", top_left_mask)
    assert np.abs(run_oracle(b) - ref).max() > 1e-3
    monkeypatch.setattr(po, "attention_request", orig)

    def gqa_modulo(q, q_pos, k_unrot, v, k_pos, q_len, base, hkv, rows=None):
        # mistake: q head h reads kv head h % Hkv instead of h // G
        hq = q.shape[1]
        G = hq // hkv
        perm = [(h % hkv) * G + h // hkv for h in range(hq)]
        inv = np.argsort(perm)
        out = orig(q[:, perm], q_pos, k_unrot, v, k_pos, q_len, base, hkv, rows)
        return out[:, inv]

    monkeypatch.setattr(po, "attention_request", gqa_modulo)
    assert np.abs(run_oracle(b) - ref).max() > 1e-3


def test_oracle_package_exports():
    for name in ["rope_frequencies", "rope_table", "rotate_half", "place_tokens",
                 "gather_request", "attention_request", "attention", "bf16_bits_to_f64"]:
        assert callable(getattr(oracle, name))

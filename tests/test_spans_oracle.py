"""Pins of the span-hashing oracle (oracle/pic_spans.py) against things other than itself.

* published FNV-1a 64 test vectors (tests/golden/fnv1a64_vectors.txt);
* closed forms of the three chaining rules of MiniPIC §2.2, written as explicit
  byte strings hashed in one go;
* the properties the page states: SSEP makes a span hash the same after any
  context; PDEP makes a block depend on the whole prompt, across SSEP restarts;
* mutation checks: planted mistakes in a copy of the rules fail these pins.
"""

import os
import struct

import numpy as np

import oracle
from oracle import pic_spans

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fnv1a64_vectors.txt")
B = 16
SSEP, PDEP = 900001, 900002


def _vectors():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        q, hx = line.rsplit(" ", 1)
        out.append((q.strip('"').encode(), int(hx, 16)))
    return out


def test_fnv1a64_published_vectors():
    vec = _vectors()
    assert len(vec) == 3
    for data, want in vec:
        assert oracle.fnv1a64(data) == want, data


def _bytes(parent, toks):
    return struct.pack("<Q", parent) + b"".join(struct.pack("<i", t) for t in toks)


def test_closed_form_chain_without_special_tokens():
    rng = np.random.default_rng(1)
    toks = rng.integers(0, 50000, size=3 * B + 5).tolist()
    seed = 0x1234
    h = oracle.block_hashes(toks, B, seed=seed)
    assert len(h) == 3  # the partial block is not hashed
    h0 = oracle.fnv1a64(_bytes(seed, toks[:B]))
    h1 = oracle.fnv1a64(_bytes(h0, toks[B:2 * B]))
    h2 = oracle.fnv1a64(_bytes(h1, toks[2 * B:3 * B]))
    assert h == [h0, h1, h2]


def test_closed_form_ssep_and_pdep():
    rng = np.random.default_rng(2)
    toks = rng.integers(0, 50000, size=5 * B).tolist()
    toks[2 * B] = SSEP
    toks[4 * B] = PDEP
    seed = 77
    h = oracle.block_hashes(toks, B, SSEP, PDEP, seed)
    a0 = oracle.fnv1a64(_bytes(seed, toks[:B]))
    a1 = oracle.fnv1a64(_bytes(a0, toks[B:2 * B]))
    a2 = oracle.fnv1a64(_bytes(seed, toks[2 * B:3 * B]))        # SSEP: chain restarts
    a3 = oracle.fnv1a64(_bytes(a2, toks[3 * B:4 * B]))
    a4 = oracle.fnv1a64(_bytes(seed, toks[:5 * B]))             # PDEP: the whole prompt
    assert h == [a0, a1, a2, a3, a4]


def test_ssep_span_hashes_the_same_after_any_context():
    rng = np.random.default_rng(3)
    span = [SSEP] + rng.integers(0, 50000, size=2 * B - 1).tolist()
    for ctx_len in [0, B, 3 * B]:
        ctx = rng.integers(0, 50000, size=ctx_len).tolist()
        h = oracle.block_hashes(ctx + span, B, SSEP, PDEP)
        assert h[ctx_len // B:] == oracle.block_hashes(span, B, SSEP, PDEP)
    # without the separator the same span hashes differently after different contexts
    plain = span[1:] + [5]
    ha = oracle.block_hashes([1] * B + plain, B)
    hb = oracle.block_hashes([2] * B + plain, B)
    assert ha[1:] != hb[1:]


def test_pdep_depends_on_the_whole_prompt_across_ssep():
    rng = np.random.default_rng(4)
    head = rng.integers(0, 50000, size=B).tolist()
    span = [SSEP] + rng.integers(0, 50000, size=B - 1).tolist()
    suffix = [PDEP] + rng.integers(0, 50000, size=B - 1).tolist()
    h1 = oracle.block_hashes(head + span + suffix, B, SSEP, PDEP)
    head2 = list(head)
    head2[3] += 1
    h2 = oracle.block_hashes(head2 + span + suffix, B, SSEP, PDEP)
    assert h1[1] == h2[1]          # the SSEP span does not see the change
    assert h1[2] != h2[2]          # the PDEP block does
    # a plain block after the SSEP span chains on the span only: it misses the change
    plain = [7] + suffix[1:]
    g1 = oracle.block_hashes(head + span + plain, B, SSEP, PDEP)
    g2 = oracle.block_hashes(head2 + span + plain, B, SSEP, PDEP)
    assert g1[2] == g2[2]


def test_special_tokens_off_the_block_start_are_ordinary():
    toks = list(range(2 * B))
    t2 = list(toks)
    t2[B + 3] = SSEP
    assert oracle.block_hashes(t2, B, SSEP, PDEP) == oracle.block_hashes(t2, B)
    assert oracle.block_hashes(t2, B, SSEP, PDEP)[1] != oracle.block_hashes(toks, B)[1]


def test_tables_share_equal_full_blocks_only():
    span = [SSEP] + list(range(1, 2 * B))
    p1 = [11] * B + span + [3, 4, 5]
    p2 = span + [PDEP] + [9] * (B - 1) + [6]
    p3 = [11] * B + span + [3, 4, 5]
    tables, k_pos, slots, nnew = oracle.build_block_tables([p1, p2, p3], B, SSEP, PDEP)
    # p1: ctx block, span (2 blocks), partial; p2: span (shared), PDEP block, partial;
    # p3 = p1: every full block shared, the partial one private
    assert tables[0] == [0, 1, 2, 3]
    assert tables[1] == [1, 2, 4, 5]
    assert tables[2] == [0, 1, 2, 6]
    assert nnew == 7
    assert k_pos[1] == list(range(len(p2)))
    assert slots[1][:2 * B] == [-1] * (2 * B)
    assert slots[2][:3 * B] == [-1] * (3 * B) and slots[2][3 * B:] == [6 * B, 6 * B + 1, 6 * B + 2]


def _mutant(kind):
    def bh(tokens, block_size, ssep=-1, pdep=-1, seed=0):
        out, parent = [], seed
        for i in range(len(tokens) // block_size):
            x = tokens[i * block_size:(i + 1) * block_size]
            if pdep >= 0 and x[0] == pdep:
                h = pic_spans._h(parent if kind == "pdep_chains" else seed,
                                 x if kind == "pdep_chains" else tokens[:(i + 1) * block_size])
            elif ssep >= 0 and x[0] == ssep and kind != "ssep_no_reset":
                h = pic_spans._h(seed, x)
            else:
                h = pic_spans._h(parent if kind != "no_chain" else seed, x)
            out.append(h)
            parent = h
        return out
    return bh


def test_planted_mistakes_fail_the_pins(monkeypatch):
    for kind, pin in [("ssep_no_reset", test_ssep_span_hashes_the_same_after_any_context),
                      ("pdep_chains", test_pdep_depends_on_the_whole_prompt_across_ssep),
                      ("no_chain", test_closed_form_chain_without_special_tokens)]:
        with monkeypatch.context() as m:
            m.setattr(oracle, "block_hashes", _mutant(kind))
            try:
                pin()
            except AssertionError:
                continue
            raise AssertionError(f"planted mistake {kind} passed its pin")

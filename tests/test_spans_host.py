"""The span-hashing host library (pic_block_hashes, pic_build_block_tables) against the
oracle: bit-exact hashes, block tables, positions and slot mappings.  Host code only."""

import numpy as np
import pytest

import oracle
import position_independent_kv_amd as pic

B = 16
SSEP, PDEP = 128001, 128002


def _compose(rng, n_spans=6, span_blocks=(1, 4), n_reqs=5, per_req=3, pad=0):
    """Prompts = a context, some SSEP spans from a shared pool (padded to blocks), a PDEP
    suffix and a ragged tail -- the composition MiniPIC §2.2 describes."""
    spans = []
    for _ in range(n_spans):
        nb = int(rng.integers(span_blocks[0], span_blocks[1] + 1))
        s = [SSEP] + rng.integers(0, 120000, size=nb * B - 1).tolist()
        spans.append(s)
    prompts = []
    for _ in range(n_reqs):
        ctx = rng.integers(0, 120000, size=int(rng.integers(0, 3)) * B).tolist()
        body = []
        for k in rng.choice(n_spans, size=per_req, replace=False):
            body += spans[int(k)]
        suffix = [PDEP] + rng.integers(0, 120000, size=B - 1).tolist()
        tail = rng.integers(0, 120000, size=int(rng.integers(0, B))).tolist()
        prompts.append(ctx + body + suffix + tail)
    return prompts


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_hashes_match_oracle(seed):
    rng = np.random.default_rng(seed)
    for p in _compose(rng):
        toks = np.asarray(p, np.int32)
        for ss, pd in [(SSEP, PDEP), (-1, -1), (SSEP, -1), (-1, PDEP)]:
            got = pic.pic_block_hashes(toks, B, ss, pd, seed=12345 + seed)
            want = oracle.block_hashes(p, B, ss, pd, seed=12345 + seed)
            assert [int(x) for x in got] == want


def test_negative_token_ids_and_odd_block_sizes():
    toks = np.asarray([-5, 7, -2147483648, 2147483647, 0, 1, 2], np.int32)
    for bs in [1, 2, 3, 7]:
        got = pic.pic_block_hashes(toks, bs, -1, -1, seed=9)
        assert [int(x) for x in got] == oracle.block_hashes(toks.tolist(), bs, seed=9)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_block_tables_match_oracle(seed):
    rng = np.random.default_rng(10 + seed)
    prompts = _compose(rng, n_reqs=7)
    cu = np.concatenate([[0], np.cumsum([len(p) for p in prompts])]).astype(np.int32)
    toks = np.concatenate([np.asarray(p, np.int32) for p in prompts])
    res = pic.pic_build_block_tables(toks, cu, B, SSEP, PDEP, seed=5, first_block=3)
    tables, k_pos, slots, nnew = oracle.build_block_tables(prompts, B, SSEP, PDEP, seed=5,
                                                           first_block=3)
    assert res["num_new_blocks"] == nnew
    for r, row in enumerate(tables):
        assert res["block_table"][r, :len(row)].tolist() == row
        assert not res["block_table"][r, len(row):].any()
    assert res["k_pos"].tolist() == sum(k_pos, [])
    assert res["slot_mapping"].tolist() == sum(slots, [])
    want_h = sum([oracle.block_hashes(p, B, SSEP, PDEP, seed=5) for p in prompts], [])
    assert [int(x) for x in res["block_hashes"]] == want_h
    # the sharing is real: fewer physical blocks than logical ones
    assert nnew < sum(-(-len(p) // B) for p in prompts)


def test_block_tables_reject_bad_arguments():
    toks = np.arange(40, dtype=np.int32)
    cu = np.asarray([0, 40], np.int32)
    with pytest.raises(pic.PicError):
        pic.pic_build_block_tables(toks, cu, block_size=8)           # kernels use 16
    with pytest.raises(pic.PicError):
        pic.pic_build_block_tables(toks, cu, num_blocks=2)           # pool too small
    with pytest.raises(pic.PicError):
        pic.pic_build_block_tables(toks, cu, stride=2)               # table too narrow
    with pytest.raises(pic.PicError):
        pic.pic_build_block_tables(toks, np.asarray([1, 40], np.int32))
    res = pic.pic_build_block_tables(toks, np.asarray([0], np.int32))
    assert res["num_new_blocks"] == 0

"""The seeded synthetic inputs: determinism, structure and bookkeeping."""

import numpy as np
import pytest
import torch

from workloads import CONFIGS, algorithmic_counts, f32_to_bf16_bits, make_workload


def test_bf16_rounding_matches_library_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -0.0, 0.0, 1e-40, -3e38, 65504.0],
                                 np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _same(a, b):
    for f in ["ctx_k", "ctx_v", "ctx_slots", "new_k", "new_v", "new_slots", "q", "cu_seqlens_q",
              "q_pos", "block_table", "seq_lens", "cu_seqlens_k", "k_pos"]:
        x, y = getattr(a, f), getattr(b, f)
        assert x.dtype == y.dtype and x.shape == y.shape and np.array_equal(x, y), f


@pytest.mark.parametrize("name", ["c1a", "c1b", "c1d"])
def test_tiny_deterministic(name):
    _same(make_workload(name), make_workload(name))


def test_resized_decode_deterministic():
    kw = dict(builder="decode", seed=2, R=8, seg_len=64, n_seg=4, n_shared=2, n_spans=4)
    _same(make_workload("x", **dict(kw)), make_workload("x", **dict(kw)))


def _written_slots(w):
    s = np.concatenate([w.ctx_slots, w.new_slots]).astype(np.int64)
    assert np.unique(s).shape[0] == s.shape[0], "a slot is written twice"
    return set(s.tolist())


@pytest.mark.parametrize("name", ["c1a", "c1b", "c1d", "c2", "c2p", "c3", "c4", "c5"])
def test_structure_invariants(name):
    w = make_workload(name, values=False)
    B = w.block_size
    written = _written_slots(w)
    assert w.cu_seqlens_k[-1] == w.k_pos.shape[0]
    assert w.cu_seqlens_q[-1] == w.q.shape[0] == w.q_pos.shape[0]
    for r in range(w.num_reqs):
        L = int(w.seq_lens[r])
        ql = int(w.cu_seqlens_q[r + 1] - w.cu_seqlens_q[r])
        assert 1 <= ql <= L
        nb = -(-L // B)
        blocks = w.block_table[r, :nb]
        assert blocks.min() >= 0 and blocks.max() < w.num_blocks
        assert np.unique(blocks).shape[0] == nb, "a block repeats inside one request"
        slots = blocks[np.arange(L) // B].astype(np.int64) * B + np.arange(L) % B
        assert set(slots.tolist()) <= written, "a visible slot is never written"
        kp = w.k_pos[w.cu_seqlens_k[r]:w.cu_seqlens_k[r] + L]
        assert kp.min() >= 0 and kp.max() < w.max_pos
        qp = w.q_pos[w.cu_seqlens_q[r]:w.cu_seqlens_q[r + 1]]
        # queries sit at the positions of the request's last q_len slots
        assert np.array_equal(qp, kp[L - ql:])


def _uses(w):
    """physical block -> set of requests referencing it."""
    u = {}
    for r in range(w.num_reqs):
        nb = -(-int(w.seq_lens[r]) // w.block_size)
        for b in w.block_table[r, :nb]:
            u.setdefault(int(b), set()).add(r)
    return u


def test_c2_sharing_pattern():
    w = make_workload("c2", values=False)
    u = _uses(w)
    shared = [b for b, rs in u.items() if len(rs) > 1]
    assert len(shared) == 32 * 64                    # 32 spans x 64 blocks
    assert all(len(u[b]) == 4 for b in shared)       # each span used by exactly 4 requests
    per_req = [sum(1 for b in w.block_table[r, :257] if len(u[int(b)]) > 1) for r in range(64)]
    assert per_req == [128] * 64                     # half of each 4096-token context shared
    # a span sits at different logical offsets in the requests that share it
    offs = {}
    for r in range(64):
        for j in range(0, 4096, 1024):
            b = int(w.block_table[r, j // 16])
            if len(u[b]) > 1:
                offs.setdefault(b, set()).add(j)
    assert sum(len(o) > 1 for o in offs.values()) > 16
    assert w.num_blocks == 10304 and np.all(w.seq_lens == 4097) and np.all(w.q_pos == 4096)


def test_c2p_has_no_sharing():
    w = make_workload("c2p", values=False)
    assert all(len(rs) == 1 for rs in _uses(w).values())
    assert w.num_blocks == 64 * 257


def test_c4_and_c5_shapes():
    w = make_workload("c4", values=False)
    assert w.num_reqs == 4 and np.all(w.seq_lens == 131073) and np.all(w.q_pos == 131072)
    sets = [set(w.block_table[r, :8192].tolist()) for r in range(4)]
    assert all(s == sets[0] for s in sets) and len(sets[0]) == 8192
    assert not np.array_equal(w.block_table[0, :8192], w.block_table[1, :8192])
    w = make_workload("c5", values=False)
    ql = w.q_lens()
    assert sorted(set(ql.tolist())) == [1, 2048]
    assert (ql == 2048).sum() == 16 and (ql == 1).sum() == 128
    assert np.all(w.seq_lens[ql == 2048] == 2048) and np.all(w.seq_lens[ql == 1] == 8193)
    assert w.total_q == 32896


def test_tiny_shares_span_at_two_offsets():
    w = make_workload("c1a")
    assert np.array_equal(w.block_table[0, :4], w.block_table[1, :4])
    assert w.block_table[0, 4] != w.block_table[1, 4]
    assert np.array_equal(w.k_pos[80:160] - w.k_pos[:80], np.full(80, 2048))
    assert np.array_equal(w.q[:16], w.q[16:]) and np.array_equal(w.new_k[:16], w.new_k[16:])
    wb = make_workload("c1b")
    assert not np.array_equal(wb.q[:16], wb.q[16:])
    wd = make_workload("c1d")
    assert wd.num_reqs == 32 and list(wd.seq_lens) == list(range(65, 81)) * 2
    assert np.array_equal(wd.q, w.q)


def test_counts_closed_forms():
    c = algorithmic_counts(make_workload("c3", values=False))
    # 8 requests x 32 heads x (512 rows x 4096 + 512*513/2) visible pairs x 4d
    assert c["flops"] == 8 * 32 * (512 * 4096 + 512 * 513 // 2) * 4 * 128
    c = algorithmic_counts(make_workload("c2", values=False))
    assert c["kv_bytes"] == 64 * 4097 * 8 * 128 * 2 * 2
    assert c["flops"] == 64 * 32 * 4097 * 4 * 128
    c = algorithmic_counts(make_workload("c1a"))
    assert c["flops"] == 2375680


def test_config_names():
    assert set(CONFIGS) == {"c1a", "c1b", "c1d", "c2", "c2p", "c3", "c4", "c5"}

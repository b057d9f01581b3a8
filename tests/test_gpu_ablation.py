"""GPU parity of the in-kernel-rotation ablation: a conventional RoPE cache
(keys rotated when they are written, one private copy per request and offset)
read by the same attention kernels with the key rotation compiled out.

The reference is the position-free oracle on the original (unrotated) batch:
attention over keys rotated to pi(j) is the same number whichever side does
the rotation (MiniPIC §2.1, Implementation: equivalent to re-rotating the
cache hit).  Tolerances as in test_gpu_parity.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_harness import DeviceWorkload, to_f64
from tests.oracle_harness import oracle_outputs, oracle_pools, select_rows
from workloads import make_workload

pytestmark = pytest.mark.gpu

TOL = 2e-2

CASES = {
    "decode": dict(builder="decode", seed=21, R=9, seg_len=96, n_seg=4, n_shared=2, n_spans=6),
    "decode_long": dict(builder="decode", seed=22, R=3, seg_len=1120, n_seg=2, n_shared=1,
                        n_spans=3),
    "decode_g8_d64": dict(builder="decode", seed=23, R=5, seg_len=64, n_seg=3, n_shared=1,
                          n_spans=5, hq=16, hkv=2, d=64),
    "prefill": dict(builder="prefill", seed=31, R=3, n_spans=5, span_len=48, per_req=2, q_len=70),
    "prefill_long_q": dict(builder="prefill", seed=32, R=2, n_spans=3, span_len=160, per_req=2,
                           q_len=300),
    "mixed": dict(builder="mixed", seed=41, n_chunks=4, chunk=96, n_dec=10, per_dec=2),
    "mixed_g2_d64": dict(builder="mixed", seed=42, n_chunks=3, chunk=160, n_dec=7, per_dec=2,
                         hq=8, hkv=4, d=64),
}


def _torch():
    import torch
    return torch


def _rotated(case):
    w = make_workload(case, **CASES[case])
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    dw.build_rotated_cache()
    return w, dw


@pytest.mark.parametrize("case,dtype", [("decode", "bf16"), ("decode_g8_d64", "bf16"),
                                        ("prefill", "f32")])
def test_cache_write_rotated_matches_oracle_rotation(case, dtype):
    """Every written key equals R_pi(j) k~_j of the oracle within the storage rounding;
    every written value equals the stored value bit for bit."""
    kw = dict(CASES[case])
    kw["dtype"] = dtype
    w = make_workload(case + "_" + dtype, **kw)
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    dw.build_rotated_cache()
    _torch().cuda.synchronize()
    kp, vp = oracle_pools(w)
    rk = dw.rot_k_pool.float().cpu().numpy().astype(np.float64)
    rv = dw.rot_v_pool.cpu()
    rv = (rv.view(_torch().int16).numpy().view(np.uint16) if dtype == "bf16"
          else rv.numpy())
    rbt = dw.rot_block_table.cpu().numpy()
    worst = 0.0
    for r in range(w.num_reqs):
        L = int(w.seq_lens[r])
        kt, vt = oracle.gather_request(kp, vp, w.block_table[r], L, w.block_size)
        kpos = w.k_pos[w.cu_seqlens_k[r]:w.cu_seqlens_k[r] + L]
        ref = oracle.rotate_half(oracle.bf16_bits_to_f64(kt) if dtype == "bf16"
                                 else kt.astype(np.float64), kpos[:, None], w.d, w.base)
        j = np.arange(L)
        got = rk[rbt[r, j // w.block_size], :, j % w.block_size, :]
        # storage rounding of the rotated key: half an ulp of the stored type, plus the fp32
        # arithmetic before it
        ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
        bound = ulp * np.maximum(np.abs(ref), 2.0 ** -30) + 1e-6
        rel = np.abs(got - ref) / bound
        worst = max(worst, float(rel.max()))
        gv = rv[rbt[r, j // w.block_size], :, :, j % w.block_size]
        assert np.array_equal(gv, vt), f"request {r}: values not copied bit for bit"
    print(f"{case}/{dtype}: worst key error {worst:.3f} of the rounding bound")
    assert worst <= 1.0


@pytest.mark.parametrize("case", sorted(CASES))
def test_rotated_cache_attention_matches_oracle(case):
    w, dw = _rotated(case)
    got = to_f64(dw.attention_rotated())
    ref = oracle_outputs(w)
    err = float(np.abs(got - ref).max())
    # the position-free kernels on the same batch
    pf = to_f64(dw.attention(out=_torch().empty_like(dw.q)))
    diff = float(np.abs(got - pf).max())
    print(f"{case}: rotated-cache max abs err {err:.3e}; vs position-free {diff:.3e}")
    assert err <= TOL
    # both paths round the same fp32 rotation to bf16 and then run identical code, so the
    # outputs are bit-identical
    assert diff == 0.0


def _rotated_named(name):
    w = make_workload(name)
    dw = DeviceWorkload(w)
    dw.write_new_tokens()
    dw.build_rotated_cache()
    return w, dw


@pytest.mark.parametrize("name", ["c3", "c2"])
def test_rotated_cache_full_size_sampled(name):
    w, dw = _rotated_named(name)
    got = to_f64(dw.attention_rotated())
    rng = np.random.default_rng(5)
    reqs = sorted(rng.choice(w.num_reqs, size=min(3, w.num_reqs), replace=False).tolist())
    rows = None
    if w.kind != "decode":
        rows = {r: sorted(rng.choice(int(w.q_lens()[r]), size=6, replace=False).tolist())
                for r in reqs}
    ref = oracle_outputs(w, requests=reqs, rows=rows)
    err = float(np.abs(select_rows(got, w, reqs, rows) - ref).max())
    print(f"{name}: rotated-cache sampled max abs err {err:.3e}")
    assert err <= TOL

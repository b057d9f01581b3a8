"""The C ABI without a GPU: symbols, host-side checks, workspace sizing, split policy.

No call here launches a kernel: every call either fails validation before any
launch or is pure host code.
"""

import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import position_independent_kv_amd as pic
from workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pic.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|void|size_t|const char\*)\s+(pic_\w+)\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = pic.library()
    names = _declared()
    assert len(names) == 32
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pic.EXPORTS)


def test_status_strings():
    for st in [0, -1, -2, -3, -4, 7]:
        assert isinstance(pic.pic_status_string(st), str)
    assert pic.pic_status_string(-3).startswith("PIC_EWORKSPACE")
    assert pic.pic_version() >= 100


def test_kernel_events_hook_arguments():
    """pic_set_kernel_events takes both handles or neither (host only, no HIP call)."""
    lib = pic.library()
    assert lib.pic_set_kernel_events(None, ctypes.c_void_p(16)) == pic.PIC_EINVAL
    assert lib.pic_set_kernel_events(ctypes.c_void_p(16), None) == pic.PIC_EINVAL
    assert lib.pic_set_kernel_events(None, None) == pic.PIC_OK
    with pytest.raises(ValueError):
        pic.pic_set_kernel_events(object(), None)


def test_timing_event_helpers_reject_null_handles():
    """The timing-event helpers check their pointers before any HIP call; destroying a null
    handle is a no-op."""
    lib = pic.library()
    assert lib.pic_timing_event_create(None) == pic.PIC_EINVAL
    assert lib.pic_timing_event_record(None, None) == pic.PIC_EINVAL
    ms = ctypes.c_float()
    assert lib.pic_timing_event_elapsed_ms(None, ctypes.c_void_p(16), ctypes.byref(ms)) \
        == pic.PIC_EINVAL
    assert lib.pic_timing_event_elapsed_ms(ctypes.c_void_p(16), None, ctypes.byref(ms)) \
        == pic.PIC_EINVAL
    assert lib.pic_timing_event_elapsed_ms(ctypes.c_void_p(16), ctypes.c_void_p(16), None) \
        == pic.PIC_EINVAL
    assert lib.pic_timing_event_destroy(None) == pic.PIC_OK


def test_workspace_size_rules():
    f = pic.pic_attn_workspace_size
    assert f(64, 64, 4097, 32, 8, 128, pic.PIC_BF16) > 0
    assert f(64, 64, 4097, 32, 8, 96, pic.PIC_BF16) == 0        # head_dim unsupported
    assert f(64, 64, 4097, 30, 8, 128, pic.PIC_BF16) == 0       # Hq % Hkv
    assert f(64, 64, 4097, 96, 2, 128, pic.PIC_BF16) == 0       # group 48 unsupported
    assert f(1, 1, 1, 4, 4, 64, 7) == 0                        # dtype
    # monotone in every bound
    a = f(8, 100, 1000, 32, 8, 128, pic.PIC_BF16)
    assert f(9, 100, 1000, 32, 8, 128, pic.PIC_BF16) >= a
    assert f(8, 200, 1000, 32, 8, 128, pic.PIC_BF16) >= a
    assert f(8, 100, 5000, 32, 8, 128, pic.PIC_BF16) >= a


SPLIT_TARGET = 512  # keys per decode chunk the library aims at (pic_common.hpp)


@pytest.mark.parametrize("dtype,kstep", [(pic.PIC_BF16, 32), (pic.PIC_F32, 16)])
def test_split_policy(dtype, kstep):
    t = SPLIT_TARGET
    prev = 1
    for L in list(range(1, 4000)) + [4097, 8193, 131073, 131072, 65537]:
        S = pic.pic_decode_num_splits(L, dtype)
        starts = [pic.pic_decode_chunk_start(L, s, dtype) for s in range(S + 1)]
        assert starts[0] == 0 and starts[-1] == L  # all keys covered, once
        assert pic.pic_decode_chunk_start(L, S + 1, dtype) == -1
        assert pic.pic_decode_chunk_start(L, -1, dtype) == -1
        assert all(x % kstep == 0 for x in starts[:-1])  # chunks start on whole steps
        lens = np.diff(starts)
        assert (lens > 0).all()                  # every chunk non-empty
        steps = -(-lens // kstep)
        assert steps.max() - steps.min() <= 1    # steps dealt out evenly
        assert steps.max() * kstep == pic.pic_decode_split_len(L, dtype)
        bound = max(1, (L + t // 2) // t)        # round(L / target): what the grid is sized by
        assert S <= bound                        # ... so no request has more chunks
        assert S == min(bound, -(-L // kstep))   # ... and no fewer, unless steps run out
        assert lens.max() <= t + t // 2 + kstep  # chunks stay near the target
        if L < 4000:
            assert bound >= prev                 # the bound never falls as L grows
            prev = bound


def _c_args(n):
    return [None] * n


def test_entry_points_reject_bad_arguments_before_launch():
    lib = pic.library()
    # rope table
    assert lib.pic_rope_table(None, None, 10, 128, 1e4, None) == pic.PIC_EINVAL
    buf = ctypes.c_void_p(1)  # never dereferenced: rejected before launch
    assert lib.pic_rope_table(buf, buf, 10, 127, 1e4, None) == pic.PIC_EUNSUPPORTED
    assert lib.pic_rope_table(buf, buf, 0, 128, 1e4, None) == pic.PIC_EINVAL
    assert lib.pic_rope_table(buf, buf, 10, 128, -1.0, None) == pic.PIC_EINVAL
    # cache write
    assert lib.pic_cache_write(None, None, None, 0, 8, 128, 1, None, None, 4, 16, None) == 0
    assert lib.pic_cache_write(None, None, None, 5, 8, 128, 1, None, None, 4, 16, None) == -1
    assert lib.pic_cache_write(buf, buf, buf, 5, 8, 128, 1, buf, buf, 4, 32, None) == -2
    assert lib.pic_cache_write(buf, buf, buf, 5, 8, 100, 1, buf, buf, 4, 16, None) == -2
    assert lib.pic_cache_write(buf, buf, buf, 5, 8, 128, 3, buf, buf, 4, 16, None) == -2
    # decode: null pointers, unsupported shapes, missing / short workspace
    args = [buf] * 5 + [300] + [buf] * 5 + [4097, 4, 32, 8, 128, 16, 100, 4097, 1] + [buf, None, 0,
                                                                                   None]
    assert lib.pic_attn_decode(*args) == pic.PIC_EWORKSPACE
    args2 = list(args)
    args2[22] = 1000  # workspace_bytes
    args2[21] = buf
    assert lib.pic_attn_decode(*args2) == pic.PIC_EWORKSPACE
    args3 = list(args)
    args3[0] = None
    assert lib.pic_attn_decode(*args3) == pic.PIC_EINVAL
    args4 = list(args)
    args4[13] = 30  # Hq not a multiple of Hkv
    assert lib.pic_attn_decode(*args4) == pic.PIC_EUNSUPPORTED
    args5 = list(args)
    args5[5] = 10  # block table too narrow for max_seq_len
    assert lib.pic_attn_decode(*args5) == pic.PIC_EINVAL
    # empty batch is a no-op
    args6 = list(args)
    args6[12] = 0
    assert lib.pic_attn_decode(*args6) == pic.PIC_OK
    # decode with append: the same checks, and both new-token rows required
    aargs = args[:1] + [buf, buf] + args[1:]
    assert lib.pic_attn_decode_append(*aargs) == pic.PIC_EWORKSPACE
    for i in (1, 2):
        bad = list(aargs)
        bad[i] = None
        assert lib.pic_attn_decode_append(*bad) == pic.PIC_EINVAL
    bad = list(aargs)
    bad[15] = 30  # Hq not a multiple of Hkv
    assert lib.pic_attn_decode_append(*bad) == pic.PIC_EUNSUPPORTED
    empty = [None, None, None] + list(args6[1:])
    empty[14] = 0
    assert lib.pic_attn_decode_append(*empty) == pic.PIC_OK
    # prefill
    pargs = [buf] * 6 + [300] + [buf] * 5 + [4097, 4, 40, 16, 32, 8, 128, 16, 100, 4097, 1] + [
        buf, None, 0, None]
    assert lib.pic_attn_prefill(*pargs) == pic.PIC_EWORKSPACE
    pargs[1] = None
    pargs[24] = buf
    pargs[25] = 1 << 40
    assert lib.pic_attn_prefill(*pargs) == pic.PIC_EINVAL


def test_shared_decode_sizes_and_rejections_before_launch():
    lib = pic.library()
    f = pic.pic_attn_decode_shared_workspace_size
    base = f(64, 4097, 32, 8, 128, pic.PIC_BF16)
    assert base > 0
    assert f(64, 4097, 32, 8, 96, pic.PIC_BF16) == 0          # head_dim unsupported
    assert f(64, 4097, 30, 8, 128, pic.PIC_BF16) == 0         # Hq % Hkv
    assert f(4, (1 << 20) + 16, 32, 8, 128, pic.PIC_BF16) == 0  # more than 65536 blocks
    assert f(4, 1 << 20, 32, 8, 128, pic.PIC_BF16) > 0        # exactly 65536 blocks
    assert f(65, 4097, 32, 8, 128, pic.PIC_BF16) >= base      # monotone
    assert f(64, 8193, 32, 8, 128, pic.PIC_BF16) >= base
    buf = ctypes.c_void_p(1)  # never dereferenced: rejected before launch
    args = [buf] * 5 + [300] + [buf] * 5 + [4097, 4, 32, 8, 128, 16, 100, 4097, 1] + [buf, None, 0,
                                                                                   None]
    assert lib.pic_attn_decode_shared(*args) == pic.PIC_EWORKSPACE
    need = f(4, 4097, 32, 8, 128, pic.PIC_BF16)  # the call's own shape: 4 requests
    assert 0 < need < base
    small = list(args)
    small[21], small[22] = buf, need - 1
    assert lib.pic_attn_decode_shared(*small) == pic.PIC_EWORKSPACE
    nulls = list(args)
    nulls[8] = None  # k_pos: the position-free kernels read it
    nulls[21], nulls[22] = buf, 1 << 40
    assert lib.pic_attn_decode_shared(*nulls) == pic.PIC_EINVAL
    big = list(args)
    big[5], big[19] = 70000, 70000 * 16  # 70000 blocks per context
    big[21], big[22] = buf, 1 << 50
    assert lib.pic_attn_decode_shared(*big) == pic.PIC_EUNSUPPORTED
    empty = list(args)
    empty[12] = 0
    assert lib.pic_attn_decode_shared(*empty) == pic.PIC_OK


def test_blocks_copy_rejects_bad_arguments_before_launch():
    lib = pic.library()
    buf = ctypes.c_void_p(1)  # never dereferenced: rejected before launch
    f = lib.pic_blocks_copy
    assert f(None, None, None, 4, None, None, None, 4, 0, 8, 128, 1, 16, None) == pic.PIC_OK
    assert f(buf, buf, None, 4, buf, buf, buf, 4, 3, 8, 128, 1, 16, None) == pic.PIC_EINVAL
    assert f(buf, buf, buf, 4, buf, buf, buf, 4, -1, 8, 128, 1, 16, None) == pic.PIC_EINVAL
    assert f(buf, buf, buf, -4, buf, buf, buf, 4, 3, 8, 128, 1, 16, None) == pic.PIC_EINVAL
    assert f(buf, buf, buf, 4, buf, buf, buf, 4, 3, 8, 96, 1, 16, None) == pic.PIC_EUNSUPPORTED
    assert f(buf, buf, buf, 4, buf, buf, buf, 4, 3, 8, 128, 5, 16, None) == pic.PIC_EUNSUPPORTED
    assert f(buf, buf, buf, 4, buf, buf, buf, 4, 3, 8, 128, 1, 32, None) == pic.PIC_EUNSUPPORTED


def test_rotated_cache_entry_points_reject_bad_arguments_before_launch():
    """The ablation entry points (rotated cache): same host checks, bf16 attention only."""
    lib = pic.library()
    buf = ctypes.c_void_p(1)  # never dereferenced: rejected before launch
    w = lib.pic_cache_write_rotated
    assert w(None, None, None, None, None, None, 10, 0, 8, 128, 1, None, None, 4, 16, None) == 0
    assert w(buf, buf, buf, None, buf, buf, 10, 5, 8, 128, 1, buf, buf, 4, 16, None) == -1
    assert w(buf, buf, buf, buf, None, buf, 10, 5, 8, 128, 1, buf, buf, 4, 16, None) == -1
    assert w(buf, buf, buf, buf, buf, buf, 0, 5, 8, 128, 1, buf, buf, 4, 16, None) == -1
    assert w(buf, buf, buf, buf, buf, buf, 10, 5, 8, 96, 1, buf, buf, 4, 16, None) == -2
    assert w(buf, buf, buf, buf, buf, buf, 10, 5, 8, 128, 1, buf, buf, 4, 8, None) == -2
    # decode over a rotated cache: 3 pointers fewer than pic_attn_decode (no k positions)
    args = [buf] * 5 + [300] + [buf] * 3 + [4097, 4, 32, 8, 128, 16, 100, 4097, 1] + [buf, None,
                                                                                   0, None]
    assert lib.pic_attn_decode_rotated(*args) == pic.PIC_EWORKSPACE
    a2 = list(args)
    a2[17] = pic.PIC_F32
    a2[19], a2[20] = buf, 1 << 40
    assert lib.pic_attn_decode_rotated(*a2) == pic.PIC_EUNSUPPORTED
    a3 = list(args)
    a3[7] = None  # cos_tab
    assert lib.pic_attn_decode_rotated(*a3) == pic.PIC_EINVAL
    a4 = list(args)
    a4[10] = 0  # empty batch
    assert lib.pic_attn_decode_rotated(*a4) == pic.PIC_OK
    pargs = [buf] * 6 + [300] + [buf] * 3 + [4097, 4, 40, 16, 32, 8, 128, 16, 100, 4097, 1] + [
        buf, None, 0, None]
    assert lib.pic_attn_prefill_rotated(*pargs) == pic.PIC_EWORKSPACE
    p2 = list(pargs)
    p2[20] = pic.PIC_F32
    p2[22], p2[23] = buf, 1 << 40
    assert lib.pic_attn_prefill_rotated(*p2) == pic.PIC_EUNSUPPORTED
    p3 = list(pargs)
    p3[1] = None
    p3[22], p3[23] = buf, 1 << 40
    assert lib.pic_attn_prefill_rotated(*p3) == pic.PIC_EINVAL


def test_validate_metadata_accepts_configs():
    for name in ["c1a", "c1d", "c2", "c3", "c4", "c5"]:
        w = make_workload(name, values=False)
        st, msg = pic.pic_validate_metadata(
            None if w.kind == "decode" else w.cu_seqlens_q, w.q_pos, w.block_table, w.seq_lens,
            w.cu_seqlens_k, w.k_pos, w.max_seq_len, w.max_pos, w.num_blocks)
        assert st == pic.PIC_OK, (name, msg)


def test_validate_metadata_catches_violations():
    w = make_workload("c1a")
    base = dict(cu_seqlens_q=w.cu_seqlens_q, q_pos=w.q_pos, block_table=w.block_table,
                seq_lens=w.seq_lens, cu_seqlens_k=w.cu_seqlens_k, k_pos=w.k_pos,
                max_seq_len=w.max_seq_len, max_pos=w.max_pos, num_blocks=w.num_blocks)

    def check(**kw):
        a = dict(base)
        a.update(kw)
        return pic.pic_validate_metadata(**a)

    assert check()[0] == pic.PIC_OK
    bt = w.block_table.copy()
    bt[1, 2] = w.num_blocks
    st, msg = check(block_table=bt)
    assert st == pic.PIC_EINVAL and "block id" in msg
    kp = w.k_pos.copy()
    kp[3] = w.max_pos
    assert "key position" in check(k_pos=kp)[1]
    qp = w.q_pos.copy()
    qp[0] = -1
    assert "query position" in check(q_pos=qp)[1]
    assert "seq_len" in check(max_seq_len=79)[1]
    sl = w.seq_lens.copy()
    sl[0] = 10
    assert check(seq_lens=sl)[0] == pic.PIC_EINVAL
    assert "stride" in check(block_table=w.block_table[:, :3])[1]


def test_host_code_under_sanitizers(tmp_path):
    """Build the host-only part with g++ -fsanitize=address,undefined and drive it."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    main = tmp_path / "main.cpp"
    main.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "pic.h"
int main() {
  int fails = 0;
  for (int s = -6; s <= 1; ++s) if (!pic_status_string(s)) ++fails;
  for (int L = 0; L < 200000; L += 37) {
    int S = pic_decode_num_splits(L, 1);
    if (L > 0 && (pic_decode_chunk_start(L, 0, 1) != 0 || pic_decode_chunk_start(L, S, 1) != L ||
                  pic_decode_chunk_start(L, S - 1, 1) >= L)) ++fails;
  }
  if (pic_attn_workspace_size(1000, 100000, 200000, 64, 8, 128, 1) == 0) ++fails;
  int cu_q[3] = {0, 2, 3}, q_pos[3] = {5, 6, 9}, bt[6] = {0, 1, 0, 2, 3, 1}, sl[2] = {7, 10};
  int cu_k[3] = {0, 7, 17}, k_pos[17];
  for (int i = 0; i < 17; ++i) k_pos[i] = i;
  char msg[64];
  if (pic_validate_metadata(cu_q, q_pos, bt, 3, sl, cu_k, k_pos, 2, 3, 10, 20, 4, 4, msg, 64) != 0) ++fails;
  bt[4] = 9;
  if (pic_validate_metadata(cu_q, q_pos, bt, 3, sl, cu_k, k_pos, 2, 3, 10, 20, 4, 4, msg, 8) == 0) ++fails;
  if (strlen(msg) > 7) ++fails;
  // span hashing and block tables: a batch with a shared SSEP span, a PDEP suffix, partial blocks
  int tok[100];
  for (int i = 0; i < 100; ++i) tok[i] = (i * 7919) % 1000;
  tok[0] = 5001; tok[50] = 5001; tok[66] = 5002;
  for (int i = 1; i < 16; ++i) tok[50 + i] = tok[i];
  unsigned long long hs[8];
  if (pic_block_hashes(tok, 100, 16, 5001, 5002, 7, (uint64_t*)hs) != 6) ++fails;
  int cu2[4] = {0, 40, 90, 100}, bt2[3 * 4], kp2[100], sm2[100], nnew = -1;
  unsigned long long bh[8];
  if (pic_build_block_tables(tok, cu2, 3, 16, 5001, 5002, 7, 0, 64, bt2, 4, kp2, sm2,
                             (uint64_t*)bh, &nnew) != 0) ++fails;
  if (nnew <= 0 || nnew > 9) ++fails;
  if (pic_build_block_tables(tok, cu2, 3, 16, 5001, 5002, 7, 0, 2, bt2, 4, kp2, sm2, NULL,
                             &nnew) == 0) ++fails;  // pool too small
  // scheduler: both policies over a trace with sharing, late arrivals and eviction
  for (int policy = 0; policy < 2; ++policy) {
    pic_sched* sc = NULL;
    if (pic_sched_create(policy, 40, 3, 24, 16, &sc) != 0 || !sc) { ++fails; continue; }
    for (int i = 0; i < 5; ++i) if (pic_sched_add_span(sc, 16 * (1 + i % 3)) != i) ++fails;
    if (pic_sched_add_span(sc, 20) >= 0) ++fails;
    for (int r = 0; r < 12; ++r) {
      int ids[3] = {r % 5, (r + 2) % 5, (r + 3) % 5};
      if (pic_sched_add_request(sc, r / 2, ids, 1 + r % 3, 5 + r, r % 4) != r) ++fails;
    }
    int cq[33], qp[64], sm[64], sl[32], ck[33], kp[4096], btab[32 * 16], kind[32], sid[32], qb[32];
    pic_sched_batch b;
    memset(&b, 0, sizeof b);
    b.max_seqs = 32; b.max_rows = 64; b.max_keys = 4096; b.block_table_stride = 16;
    b.cu_seqlens_q = cq; b.q_pos = qp; b.slot_mapping = sm; b.seq_lens = sl; b.cu_seqlens_k = ck;
    b.k_pos = kp; b.block_table = btab; b.seq_kind = kind; b.seq_id = sid; b.q_begin = qb;
    int st, steps = 0, done = 0;
    while ((st = pic_sched_step(sc, &b)) == 1 && steps < 10000) {
      ++steps;
      done += b.num_finished;
      if (b.total_q > 40 || b.cu_seqlens_q[b.num_seqs] != b.total_q) ++fails;
    }
    if (st != 0 || done != 12) ++fails;
    b.max_rows = 0;
    if (pic_sched_step(sc, &b) != 0) ++fails;  // finished: no arrays needed
    pic_sched_destroy(sc);
  }
  printf("fails=%d\n", fails);
  return fails;
}
''')
    exe = tmp_path / "host_test"
    csrc = os.path.join(ROOT, "position_independent_kv_amd", "csrc")
    srcs = [os.path.join(csrc, n) for n in ("pic_host.cpp", "pic_spans.cpp", "pic_sched.cpp")]
    cmd = [gxx, "-std=c++17", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), *srcs, str(main), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "fails=0" in res.stdout


C_CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "pic.h"

int main(void) {
    int32_t tokens[40];
    uint64_t h1[2], h2[2];
    int i, n;
    for (i = 0; i < 40; ++i) tokens[i] = 1000 + i;
    if (pic_version() <= 0) return 1;
    if (strncmp(pic_status_string(PIC_EWORKSPACE), "PIC_EWORKSPACE", 14) != 0) return 2;
    if (pic_attn_workspace_size(64, 64, 4097, 32, 8, 128, PIC_BF16) == 0) return 3;
    if (pic_decode_num_splits(4097, PIC_BF16) < 1) return 4;
    /* two full blocks of 16 tokens, the 8-token tail is not hashed */
    n = pic_block_hashes(tokens, 40, 16, -1, -1, 7u, h1);
    if (n != 2) return 5;
    if (pic_block_hashes(tokens, 40, 16, -1, -1, 7u, h2) != 2) return 6;
    if (h1[0] != h2[0] || h1[1] != h2[1] || h1[0] == h1[1]) return 7;
    /* an attention call with a null workspace is rejected before any launch */
    if (pic_attn_decode(tokens, tokens, tokens, tokens, tokens, 1, tokens, tokens, tokens,
                        (const float*)tokens, (const float*)tokens, 8, 1, 4, 4, 64, 16, 1, 16,
                        PIC_F32, tokens, NULL, 0, NULL) != PIC_EWORKSPACE) return 8;
    printf("ok %d\n", pic_version());
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_header_is_c99_and_the_library_links_from_c(tmp_path):
    """The boundary is a C ABI: include/pic.h compiles as strict C99 and a C program linked
    against libpic.so calls its host-side entry points (no GPU work)."""
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    lib_dir = os.path.dirname(pic.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
           os.path.join(ROOT, "include"), str(src), "-L", lib_dir, "-lpic",
           f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    if not os.path.exists(os.path.join(lib_dir, "libpic.so")):
        pytest.skip("libpic.so is not built")
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert run.stdout.startswith("ok ")


# ---------------------------------------------------------------------------
# the Python binding's own checks (no device memory involved: CPU tensors fail
# the checks before any pointer is taken)
# ---------------------------------------------------------------------------

def _cpu_decode_args(w):
    import torch

    def t(a):
        return torch.from_numpy(np.array(a, dtype=np.int32))  # a copy: tests mutate it

    q = torch.zeros((w.num_reqs, w.hq, w.d), dtype=torch.bfloat16)
    kp = torch.zeros((w.num_blocks, w.hkv, w.block_size, w.d), dtype=torch.bfloat16)
    vp = torch.zeros((w.num_blocks, w.hkv, w.d, w.block_size), dtype=torch.bfloat16)
    cos = torch.zeros((w.max_pos, w.d // 2))
    return dict(q=q, q_pos=t(w.q_pos), k_pool=kp, v_pool=vp, block_table=t(w.block_table),
                seq_lens=t(w.seq_lens), cu_seqlens_k=t(w.cu_seqlens_k), k_pos=t(w.k_pos),
                cos_tab=cos, sin_tab=cos.clone(), max_seq_len=w.max_seq_len,
                out=torch.zeros_like(q), workspace=torch.zeros(16, dtype=torch.uint8))


def test_binding_rejects_short_metadata_and_wrong_table_width():
    """Every array the kernels index must have the length the call implies, and the table
    must be built for this head size: a table of d/2 = 32 columns read as d = 128 would put
    every row lookup past its end on the device."""
    import torch
    w = make_workload("x", values=False, builder="decode", seed=3, R=4, seg_len=32, n_seg=2,
                      n_shared=0, n_spans=0)
    good = _cpu_decode_args(w)
    bad = {
        "cos_tab": torch.zeros((w.max_pos, 32)),
        "q_pos": good["q_pos"][:-1],
        "seq_lens": good["seq_lens"][:-1],
        "cu_seqlens_k": good["cu_seqlens_k"][:-1],
        "block_table": good["block_table"][:-1],
        "k_pos": good["k_pos"].view(2, -1),
    }
    for name, val in bad.items():
        kw = dict(good)
        kw[name] = val
        if name == "cos_tab":
            kw["sin_tab"] = val.clone()
        with pytest.raises(ValueError) as e:
            pic.pic_attn_decode(**kw)
        assert "must be on the GPU" not in str(e.value), name
    # with good shapes the first complaint is that the tensors are not on the GPU
    with pytest.raises(ValueError, match="GPU"):
        pic.pic_attn_decode(**good)


def test_binding_validate_mode_checks_device_values(monkeypatch):
    """PIC_VALIDATE=1: the binding copies the metadata to the host and runs
    pic_validate_metadata (plus the k_pos length and max_q_len) before launching."""
    w = make_workload("x", values=False, builder="decode", seed=3, R=4, seg_len=32, n_seg=2,
                      n_shared=0, n_spans=0)
    monkeypatch.setenv("PIC_VALIDATE", "1")
    good = _cpu_decode_args(w)
    with pytest.raises(ValueError, match="GPU"):  # valid metadata: on to the pointer checks
        pic.pic_attn_decode(**good)
    cases = {
        "block id": ("block_table", lambda a: a.fill_(w.num_blocks)),
        "key position": ("k_pos", lambda a: a.__setitem__(5, w.max_pos)),
        "query position": ("q_pos", lambda a: a.__setitem__(0, -1)),
        "seq_len": ("seq_lens", lambda a: a.__setitem__(1, w.max_seq_len + 1)),
        "k_pos holds": ("k_pos", None),
    }
    for what, (name, mutate) in cases.items():
        kw = _cpu_decode_args(w)
        if mutate is None:
            kw[name] = kw[name][:-3].clone()
        else:
            mutate(kw[name])
        with pytest.raises(ValueError, match=what):
            pic.pic_attn_decode(**kw)
    # decode with append: the block receiving a request's new token must be its own
    kw = _cpu_decode_args(w)
    new = kw["q"].new_zeros((w.num_reqs, w.hkv, w.d))
    app = dict(kw, new_k=new, new_v=new.clone())
    with pytest.raises(ValueError, match="GPU"):
        pic.pic_attn_decode_append(**app)
    bt = app["block_table"]
    L1 = int(app["seq_lens"][1])
    bt[1, (L1 - 1) // w.block_size] = bt[0, 0]   # request 1's tail block is request 0's first
    with pytest.raises(ValueError, match="request 1 appends to block"):
        pic.pic_attn_decode_append(**app)
    # prefill: a request longer than max_q_len
    import torch
    pw = make_workload("y", values=False, builder="prefill", seed=4, R=2, n_spans=3, span_len=32,
                       per_req=2, q_len=20)
    a = _cpu_decode_args(pw)
    q = torch.zeros((pw.total_q, pw.hq, pw.d), dtype=torch.bfloat16)
    cu_q = torch.from_numpy(pw.cu_seqlens_q.copy())
    args = (q, cu_q, a["q_pos"], a["k_pool"], a["v_pool"], a["block_table"], a["seq_lens"],
            a["cu_seqlens_k"], a["k_pos"], a["cos_tab"], a["sin_tab"])
    with pytest.raises(ValueError, match="max_q_len"):
        pic.pic_attn_prefill(*args, 19, pw.max_seq_len, torch.zeros_like(q), a["workspace"])
    with pytest.raises(ValueError, match="GPU"):
        pic.pic_attn_prefill(*args, 20, pw.max_seq_len, torch.zeros_like(q), a["workspace"])


def test_stream_read_rejects_bad_arguments_before_launch():
    lib = pic.library()
    p = ctypes.c_void_p(4096)
    f = lib.pic_stream_read
    assert f(None, 1 << 20, None, 0, 64, p, None) == pic.PIC_EINVAL
    assert f(p, 1 << 20, None, 0, 64, None, None) == pic.PIC_EINVAL
    assert f(p, 0, None, 0, 64, p, None) == pic.PIC_EINVAL
    assert f(p, 1000, None, 0, 64, p, None) == pic.PIC_EINVAL           # not 4 KiB segments
    assert f(p, 1 << 20, None, 0, 0, p, None) == pic.PIC_EINVAL
    assert f(p, 1 << 20, None, 0, (1 << 20) + 1, p, None) == pic.PIC_EINVAL
    assert f(p, 1 << 20, p, 0, 64, p, None) == pic.PIC_EINVAL            # pieces need a size
    assert f(p, 1 << 20, p, 6144, 64, p, None) == pic.PIC_EINVAL         # not 4 KiB multiples
    assert f(p, 3 << 12, p, 8192, 64, p, None) == pic.PIC_EINVAL         # does not divide bytes

"""Position-free paged attention for MI355X (gfx950): Python binding.

Thin ctypes marshalling over ``libpic.so`` (declared in ``include/pic.h``):
each function takes torch tensors, checks dtypes / shapes / devices, derives
the integer sizes from the shapes, and passes raw pointers plus the current
HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no fallback path.  If the library is not built, importing
works but every call raises ``PicLibraryMissing``.

The operation is the one of "MiniPIC: Flexible Position-Independent Caching
in <100LOC", §2.1: keys cached unrotated, rotary rotation applied inside the
attention kernel from each request's logical positions.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# PIC_LIBRARY may name another build of the same library (same ABI).
LIB_PATH = os.environ.get("PIC_LIBRARY") or os.path.join(HERE, "libpic.so")

PIC_OK, PIC_EINVAL, PIC_EUNSUPPORTED, PIC_EWORKSPACE, PIC_EHIP = 0, -1, -2, -3, -4
PIC_F32, PIC_BF16 = 0, 1
BLOCK_SIZE = 16

EXPORTS = [
    "pic_status_string", "pic_version", "pic_rope_table", "pic_cache_write",
    "pic_attn_workspace_size", "pic_attn_decode", "pic_attn_prefill", "pic_validate_metadata",
    "pic_decode_num_splits", "pic_decode_chunk_start", "pic_decode_split_len",
    "pic_cache_write_rotated",
    "pic_attn_decode_rotated", "pic_attn_prefill_rotated", "pic_block_hashes",
    "pic_build_block_tables", "pic_blocks_copy", "pic_sched_create", "pic_sched_destroy",
    "pic_sched_add_span", "pic_sched_add_request", "pic_sched_step", "pic_set_kernel_events",
    "pic_attn_decode_shared", "pic_attn_decode_shared_workspace_size", "pic_attn_decode_noalloc",
    "pic_stream_read", "pic_attn_decode_append", "pic_timing_event_create",
    "pic_timing_event_record", "pic_timing_event_elapsed_ms", "pic_timing_event_destroy",
]
PIC_SCHED_ISPS, PIC_SCHED_BARRIER = 0, 1
PIC_SEQ_SPAN, PIC_SEQ_PROMPT, PIC_SEQ_DECODE = 0, 1, 2


class PicError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_status_string(status)} ({status})")


class PicLibraryMissing(RuntimeError):
    pass


class _SchedBatch(ctypes.Structure):
    """pic_sched_batch (include/pic.h), field for field."""
    _fields_ = [
        ("max_seqs", ctypes.c_int), ("max_rows", ctypes.c_int), ("max_keys", ctypes.c_longlong),
        ("block_table_stride", ctypes.c_int),
        *[(n, ctypes.c_void_p) for n in ("cu_seqlens_q", "q_pos", "slot_mapping", "seq_lens",
                                         "cu_seqlens_k", "k_pos", "block_table", "seq_kind",
                                         "seq_id", "q_begin")],
        ("step", ctypes.c_longlong), ("num_seqs", ctypes.c_int), ("total_q", ctypes.c_int),
        ("max_q_len", ctypes.c_int), ("max_seq_len", ctypes.c_int),
        ("total_keys", ctypes.c_longlong), ("num_finished", ctypes.c_int),
    ]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise PicLibraryMissing(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_void, c_size, c_double = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_double
    c_char_p = ctypes.c_char_p
    lib.pic_status_string.restype = c_char_p
    lib.pic_status_string.argtypes = [c_int]
    lib.pic_version.restype = c_int
    lib.pic_rope_table.argtypes = [c_void, c_void, c_int, c_int, c_double, c_void]
    lib.pic_cache_write.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_void,
                                    c_void, c_int, c_int, c_void]
    lib.pic_attn_workspace_size.restype = c_size
    lib.pic_attn_workspace_size.argtypes = [c_int] * 7
    lib.pic_attn_decode.argtypes = ([c_void] * 5 + [c_int] + [c_void] * 5 + [c_int] * 9
                                    + [c_void, c_void, c_size, c_void])
    lib.pic_attn_prefill.argtypes = ([c_void] * 6 + [c_int] + [c_void] * 5 + [c_int] * 11
                                     + [c_void, c_void, c_size, c_void])
    lib.pic_validate_metadata.argtypes = ([c_void] * 3 + [c_int] + [c_void] * 3 + [c_int] * 6
                                          + [ctypes.c_char_p, c_int])
    lib.pic_cache_write_rotated.argtypes = ([c_void] * 6 + [c_int] * 5 + [c_void, c_void]
                                            + [c_int, c_int, c_void])
    lib.pic_attn_decode_rotated.argtypes = ([c_void] * 5 + [c_int] + [c_void] * 3 + [c_int] * 9
                                            + [c_void, c_void, c_size, c_void])
    lib.pic_attn_prefill_rotated.argtypes = ([c_void] * 6 + [c_int] + [c_void] * 3
                                             + [c_int] * 11 + [c_void, c_void, c_size, c_void])
    c_i32, c_u64 = ctypes.c_int32, ctypes.c_uint64
    lib.pic_block_hashes.argtypes = [c_void, c_int, c_int, c_i32, c_i32, c_u64, c_void]
    lib.pic_build_block_tables.argtypes = ([c_void, c_void, c_int, c_int, c_i32, c_i32, c_u64,
                                            c_int, c_int, c_void, c_int, c_void, c_void, c_void,
                                            c_void])
    lib.pic_blocks_copy.argtypes = ([c_void] * 3 + [c_int] + [c_void] * 3 + [c_int] * 6
                                    + [c_void])
    lib.pic_sched_create.argtypes = [c_int] * 5 + [ctypes.POINTER(c_void)]
    lib.pic_sched_destroy.restype = None
    lib.pic_sched_destroy.argtypes = [c_void]
    lib.pic_sched_add_span.argtypes = [c_void, c_int]
    lib.pic_sched_add_request.argtypes = [c_void, ctypes.c_longlong, c_void, c_int, c_int, c_int]
    lib.pic_sched_step.argtypes = [c_void, ctypes.POINTER(_SchedBatch)]
    lib.pic_set_kernel_events.argtypes = [c_void, c_void]
    lib.pic_attn_decode_shared.argtypes = lib.pic_attn_decode.argtypes
    lib.pic_timing_event_create.argtypes = [ctypes.POINTER(c_void)]
    lib.pic_timing_event_record.argtypes = [c_void, c_void]
    lib.pic_timing_event_elapsed_ms.argtypes = [c_void, c_void, ctypes.POINTER(ctypes.c_float)]
    lib.pic_timing_event_destroy.argtypes = [c_void]
    lib.pic_attn_decode_append.argtypes = ([c_void] * 7 + [c_int] + [c_void] * 5 + [c_int] * 9
                                           + [c_void, c_void, c_size, c_void])
    lib.pic_attn_decode_noalloc.argtypes = ([c_void] * 5 + [c_int] + [c_void] * 5 + [c_int] * 9
                                            + [c_void, c_void])
    lib.pic_attn_decode_shared_workspace_size.restype = c_size
    lib.pic_attn_decode_shared_workspace_size.argtypes = [c_int] * 6
    lib.pic_stream_read.argtypes = [c_void, c_size, c_void, c_int, c_int, c_void, c_void]
    lib.pic_decode_num_splits.argtypes = [c_int, c_int]
    lib.pic_decode_split_len.argtypes = [c_int, c_int]
    lib.pic_decode_chunk_start.argtypes = [c_int, c_int, c_int]
    for name in EXPORTS:
        getattr(lib, name)  # every declared symbol must resolve
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises PicLibraryMissing if not built)."""
    return _load()


def _status_string(status: int) -> str:
    try:
        return _load().pic_status_string(status).decode()
    except PicLibraryMissing:
        return "status"


def _check(status: int, where: str):
    if status != PIC_OK:
        raise PicError(status, where)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PIC_BF16
    if t.dtype == torch.float32:
        return PIC_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t, name, dtype=None):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def pic_version() -> int:
    return _load().pic_version()


def pic_status_string(status: int) -> str:
    return _load().pic_status_string(status).decode()


def pic_rope_table(cos_tab, sin_tab, base: float, stream=None):
    """Fill float32 [max_pos][head_dim/2] cos/sin tables for rotary base ``base``."""
    torch = _torch()
    if cos_tab.shape != sin_tab.shape or cos_tab.dim() != 2:
        raise ValueError("cos_tab and sin_tab must both be [max_pos][head_dim/2]")
    max_pos, half = cos_tab.shape
    _check(_load().pic_rope_table(_ptr(cos_tab, "cos_tab", torch.float32),
                                  _ptr(sin_tab, "sin_tab", torch.float32), max_pos, 2 * half,
                                  float(base), _stream(stream)), "pic_rope_table")


def pic_cache_write(k, v, slot_mapping, k_pool, v_pool, stream=None):
    """Scatter unrotated k, v [T][Hkv][d] into the pools at slot_mapping[T] (int32)."""
    torch = _torch()
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must both be [num_tokens][Hkv][head_dim]")
    T, hkv, d = k.shape
    nb, phkv, bs, pd = k_pool.shape
    if (phkv, pd) != (hkv, d) or tuple(v_pool.shape) != (nb, hkv, d, bs):
        raise ValueError("pool shapes must be k [nb][Hkv][B][d] and v [nb][Hkv][d][B]")
    if k.dtype != k_pool.dtype or v.dtype != k.dtype or v_pool.dtype != k.dtype:
        raise TypeError("k, v and the pools must share one dtype")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    _check(_load().pic_cache_write(_ptr(k, "k"), _ptr(v, "v"),
                                   _ptr(slot_mapping, "slot_mapping", torch.int32), T, hkv, d,
                                   _dtype_code(k), _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"),
                                   nb, bs, _stream(stream)), "pic_cache_write")


def pic_cache_write_rotated(k, v, slot_mapping, positions, cos_tab, sin_tab, k_pool, v_pool,
                            stream=None):
    """Conventional RoPE-cache write (ablation baseline): store R_pos k and v at slot_mapping."""
    torch = _torch()
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must both be [num_tokens][Hkv][head_dim]")
    T, hkv, d = k.shape
    nb, phkv, bs, pd = k_pool.shape
    if (phkv, pd) != (hkv, d) or tuple(v_pool.shape) != (nb, hkv, d, bs):
        raise ValueError("pool shapes must be k [nb][Hkv][B][d] and v [nb][Hkv][d][B]")
    if k.dtype != k_pool.dtype or v.dtype != k.dtype or v_pool.dtype != k.dtype:
        raise TypeError("k, v and the pools must share one dtype")
    if slot_mapping.shape != (T,) or positions.shape != (T,):
        raise ValueError("slot_mapping and positions must be [num_tokens]")
    if cos_tab.shape != sin_tab.shape or cos_tab.dim() != 2 or 2 * cos_tab.shape[1] != d:
        raise ValueError("cos_tab and sin_tab must both be [max_pos][head_dim/2]")
    _check(_load().pic_cache_write_rotated(
        _ptr(k, "k"), _ptr(v, "v"), _ptr(slot_mapping, "slot_mapping", torch.int32),
        _ptr(positions, "positions", torch.int32), _ptr(cos_tab, "cos_tab", torch.float32),
        _ptr(sin_tab, "sin_tab", torch.float32), cos_tab.shape[0], T, hkv, d, _dtype_code(k),
        _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"), nb, bs, _stream(stream)),
        "pic_cache_write_rotated")


def pic_attn_workspace_size(num_reqs, total_q, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                            dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return int(_load().pic_attn_workspace_size(num_reqs, total_q, max_seq_len, num_q_heads,
                                               num_kv_heads, head_dim, code))


def _pool_dims(k_pool, v_pool):
    nb, hkv, bs, d = k_pool.shape
    if tuple(v_pool.shape) != (nb, hkv, d, bs):
        raise ValueError("v_pool must be [num_blocks][Hkv][head_dim][block_size]")
    return nb, hkv, bs, d


def pic_attn_decode(q, q_pos, k_pool, v_pool, block_table, seq_lens, cu_seqlens_k, k_pos,
                    cos_tab, sin_tab, max_seq_len, out, workspace, stream=None):
    """One query row per request: q, out [R][Hq][d]; metadata int32 device tensors."""
    _decode_call("pic_attn_decode", q, q_pos, k_pool, v_pool, block_table, seq_lens,
                 cu_seqlens_k, k_pos, cos_tab, sin_tab, max_seq_len, out, workspace, stream)


def pic_attn_decode_append(q, new_k, new_v, q_pos, k_pool, v_pool, block_table, seq_lens,
                           cu_seqlens_k, k_pos, cos_tab, sin_tab, max_seq_len, out, workspace,
                           stream=None):
    """pic_attn_decode that also writes each request's new token: new_k, new_v [R][Hkv][d]
    (q's dtype) are request r's key (unrotated) and value, stored as its key slot
    seq_lens[r] - 1, which the same call attends to.  The pools hold the same bytes and out
    the same values as pic_cache_write followed by pic_attn_decode."""
    torch = _torch()
    i32 = torch.int32
    fn = "pic_attn_decode_append"
    R, hq, d = q.shape
    nb, hkv, bs, pd = _pool_dims(k_pool, v_pool)
    if pd != d or tuple(out.shape) != (R, hq, d) or out.dtype != q.dtype:
        raise ValueError("q / out / pool head sizes disagree")
    for t in (new_k, new_v):
        if tuple(t.shape) != (R, hkv, d):
            raise ValueError(f"{fn}: new_k / new_v must be [{R}][{hkv}][{d}]")
    _check_meta(fn, R, R, d, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos, cos_tab, sin_tab)
    if validation_enabled():
        _validate(fn, None, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos, 1, max_seq_len,
                  cos_tab.shape[0], nb)
        _validate_append(fn, block_table, seq_lens, bs)
    _check(_load().pic_attn_decode_append(
        _ptr(q, "q"), _ptr(new_k, "new_k", q.dtype), _ptr(new_v, "new_v", q.dtype),
        _ptr(q_pos, "q_pos", i32), _ptr(k_pool, "k_pool", q.dtype),
        _ptr(v_pool, "v_pool", q.dtype), _ptr(block_table, "block_table", i32),
        block_table.shape[1], _ptr(seq_lens, "seq_lens", i32),
        _ptr(cu_seqlens_k, "cu_seqlens_k", i32), _ptr(k_pos, "k_pos", i32),
        _ptr(cos_tab, "cos_tab", torch.float32), _ptr(sin_tab, "sin_tab", torch.float32),
        cos_tab.shape[0], R, hq, hkv, d, bs, nb, int(max_seq_len), _dtype_code(q),
        _ptr(out, "out"), _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), fn)


def pic_attn_decode_shared(q, q_pos, k_pool, v_pool, block_table, seq_lens, cu_seqlens_k,
                           k_pos, cos_tab, sin_tab, max_seq_len, out, workspace, stream=None):
    """pic_attn_decode with block-determined chunks, identical chunks co-scheduled on one XCD;
    the workspace is sized by pic_attn_decode_shared_workspace_size."""
    _decode_call("pic_attn_decode_shared", q, q_pos, k_pool, v_pool, block_table, seq_lens,
                 cu_seqlens_k, k_pos, cos_tab, sin_tab, max_seq_len, out, workspace, stream)


def pic_attn_decode_noalloc(q, q_pos, k_pool, v_pool, block_table, seq_lens, cu_seqlens_k,
                            k_pos, cos_tab, sin_tab, max_seq_len, out, stream=None):
    """pic_attn_decode without a workspace argument: the chunk partials live in the
    library's fixed per-device scratch array (64 MiB), so the call allocates nothing.
    Calls that overlap in time on one GPU race on that array."""
    torch = _torch()
    i32 = torch.int32
    fn = "pic_attn_decode_noalloc"
    R, hq, d = q.shape
    nb, hkv, bs, pd = _pool_dims(k_pool, v_pool)
    if pd != d or tuple(out.shape) != (R, hq, d) or out.dtype != q.dtype:
        raise ValueError("q / out / pool head sizes disagree")
    _check_meta(fn, R, R, d, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos, cos_tab, sin_tab)
    if validation_enabled():
        _validate(fn, None, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos, 1, max_seq_len,
                  cos_tab.shape[0], nb)
    _check(_load().pic_attn_decode_noalloc(
        _ptr(q, "q"), _ptr(q_pos, "q_pos", i32), _ptr(k_pool, "k_pool", q.dtype),
        _ptr(v_pool, "v_pool", q.dtype), _ptr(block_table, "block_table", i32),
        block_table.shape[1], _ptr(seq_lens, "seq_lens", i32),
        _ptr(cu_seqlens_k, "cu_seqlens_k", i32), _ptr(k_pos, "k_pos", i32),
        _ptr(cos_tab, "cos_tab", torch.float32), _ptr(sin_tab, "sin_tab", torch.float32),
        cos_tab.shape[0], R, hq, hkv, d, bs, nb, int(max_seq_len), _dtype_code(q),
        _ptr(out, "out"), _stream(stream)), fn)


def pic_attn_decode_shared_workspace_size(num_reqs, max_seq_len, num_q_heads, num_kv_heads,
                                          head_dim, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return int(_load().pic_attn_decode_shared_workspace_size(
        num_reqs, max_seq_len, num_q_heads, num_kv_heads, head_dim, code))


def _check_meta(fn, R, total_q, d, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos, cos_tab,
                sin_tab, cu_seqlens_q=None):
    """Shapes of the metadata and the table (no device reads): every length the kernels
    index by must be there, and the table must be built for this head size."""
    if cos_tab.shape != sin_tab.shape or cos_tab.dim() != 2 or 2 * cos_tab.shape[1] != d:
        raise ValueError(f"{fn}: cos_tab and sin_tab must both be [max_pos][{d // 2}]")
    if q_pos.dim() != 1 or q_pos.shape[0] != total_q:
        raise ValueError(f"{fn}: q_pos must be [{total_q}]")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != R:
        raise ValueError(f"{fn}: seq_lens must be [{R}]")
    if block_table.dim() != 2 or block_table.shape[0] < R:
        raise ValueError(f"{fn}: block_table must be [R][stride]")
    if cu_seqlens_k is not None and (cu_seqlens_k.dim() != 1 or cu_seqlens_k.shape[0] != R + 1):
        raise ValueError(f"{fn}: cu_seqlens_k must be [{R + 1}]")
    if k_pos is not None and k_pos.dim() != 1:
        raise ValueError(f"{fn}: k_pos must be one-dimensional")
    if cu_seqlens_q is not None and (cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape[0] != R + 1):
        raise ValueError(f"{fn}: cu_seqlens_q must be [{R + 1}]")


def validation_enabled() -> bool:
    """PIC_VALIDATE=1: every attention call first checks its metadata on host copies."""
    return os.environ.get("PIC_VALIDATE", "") == "1"


def _validate(fn, cu_seqlens_q, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos, max_q_len,
              max_seq_len, max_pos, num_blocks):
    """The device-value preconditions of an attention call, checked on host copies (this
    synchronises with the device).  Raises ValueError naming the first violation."""
    host = [None if t is None else t.detach().cpu().numpy()
            for t in (cu_seqlens_q, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos)]
    cu_q, qp, bt, sl, cu_k, kp = host
    R = sl.shape[0]
    if cu_k is not None and R and kp.shape[0] < int(cu_k[R]):
        raise ValueError(f"{fn}: k_pos holds {kp.shape[0]} entries, cu_seqlens_k[R] = {cu_k[R]}")
    if cu_k is None:  # a rotated-cache call: positions are not read, any in-range value will do
        cu_k = np.concatenate([[0], np.cumsum(sl.astype(np.int64))]).astype(np.int32)
        kp = np.zeros(int(cu_k[-1]), np.int32)
    st, msg = pic_validate_metadata(cu_q, qp, bt[:R], sl, cu_k, kp, max_seq_len, max_pos,
                                    num_blocks)
    if st != PIC_OK:
        raise ValueError(f"{fn}: {msg}")
    if cu_q is not None and R and int(np.diff(cu_q.astype(np.int64)).max()) > max_q_len:
        raise ValueError(f"{fn}: a request has more than max_q_len = {max_q_len} query rows")


def _validate_append(fn, block_table, seq_lens, block_size):
    """pic_attn_decode_append's own precondition, on host copies: the block that receives a
    request's new token (its key slot seq_lens[r] - 1) is read by no other request of the
    call (the launch writes it while the other requests' chunks read theirs)."""
    bt = block_table.detach().cpu().numpy()
    sl = seq_lens.detach().cpu().numpy().astype(np.int64)
    R = sl.shape[0]
    nb = (np.maximum(sl, 0) + block_size - 1) // block_size
    owner = np.repeat(np.arange(R), nb)
    used = np.concatenate([bt[r, :nb[r]] for r in range(R)]) if R else np.zeros(0, np.int64)
    for r in np.flatnonzero(sl > 0):
        tail = bt[r, (sl[r] - 1) // block_size]
        others = owner[(used == tail) & (owner != r)]
        if others.size:
            raise ValueError(f"{fn}: request {r} appends to block {tail}, which request "
                             f"{int(others[0])} also reads")


def _decode_call(fn, q, q_pos, k_pool, v_pool, block_table, seq_lens, cu_seqlens_k, k_pos,
                 cos_tab, sin_tab, max_seq_len, out, workspace, stream):
    torch = _torch()
    i32 = torch.int32
    R, hq, d = q.shape
    nb, hkv, bs, pd = _pool_dims(k_pool, v_pool)
    if pd != d or tuple(out.shape) != (R, hq, d) or out.dtype != q.dtype:
        raise ValueError("q / out / pool head sizes disagree")
    _check_meta(fn, R, R, d, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos, cos_tab, sin_tab)
    if validation_enabled():
        _validate(fn, None, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos, 1, max_seq_len,
                  cos_tab.shape[0], nb)
    _check(getattr(_load(), fn)(
        _ptr(q, "q"), _ptr(q_pos, "q_pos", i32), _ptr(k_pool, "k_pool", q.dtype),
        _ptr(v_pool, "v_pool", q.dtype), _ptr(block_table, "block_table", i32),
        block_table.shape[1], _ptr(seq_lens, "seq_lens", i32),
        _ptr(cu_seqlens_k, "cu_seqlens_k", i32), _ptr(k_pos, "k_pos", i32),
        _ptr(cos_tab, "cos_tab", torch.float32), _ptr(sin_tab, "sin_tab", torch.float32),
        cos_tab.shape[0], R, hq, hkv, d, bs, nb, int(max_seq_len), _dtype_code(q),
        _ptr(out, "out"), _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), fn)


def pic_attn_prefill(q, cu_seqlens_q, q_pos, k_pool, v_pool, block_table, seq_lens,
                     cu_seqlens_k, k_pos, cos_tab, sin_tab, max_q_len, max_seq_len, out,
                     workspace, stream=None):
    """Mixed batch in one launch: q, out [total_q][Hq][d]; cu_seqlens_q [R+1]."""
    torch = _torch()
    i32 = torch.int32
    total_q, hq, d = q.shape
    R = seq_lens.shape[0]
    nb, hkv, bs, pd = _pool_dims(k_pool, v_pool)
    if pd != d or tuple(out.shape) != (total_q, hq, d) or out.dtype != q.dtype:
        raise ValueError("q / out / pool head sizes disagree")
    _check_meta("pic_attn_prefill", R, total_q, d, q_pos, block_table, seq_lens, cu_seqlens_k,
                k_pos, cos_tab, sin_tab, cu_seqlens_q)
    if validation_enabled():
        _validate("pic_attn_prefill", cu_seqlens_q, q_pos, block_table, seq_lens, cu_seqlens_k,
                  k_pos, int(max_q_len), max_seq_len, cos_tab.shape[0], nb)
    _check(_load().pic_attn_prefill(
        _ptr(q, "q"), _ptr(cu_seqlens_q, "cu_seqlens_q", i32), _ptr(q_pos, "q_pos", i32),
        _ptr(k_pool, "k_pool", q.dtype), _ptr(v_pool, "v_pool", q.dtype),
        _ptr(block_table, "block_table", i32), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", i32), _ptr(cu_seqlens_k, "cu_seqlens_k", i32),
        _ptr(k_pos, "k_pos", i32), _ptr(cos_tab, "cos_tab", torch.float32),
        _ptr(sin_tab, "sin_tab", torch.float32), cos_tab.shape[0], R, total_q, int(max_q_len),
        hq, hkv, d, bs, nb, int(max_seq_len), _dtype_code(q), _ptr(out, "out"),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), "pic_attn_prefill")


def pic_attn_decode_rotated(q, q_pos, k_pool, v_pool, block_table, seq_lens, cos_tab, sin_tab,
                            max_seq_len, out, workspace, stream=None):
    """pic_attn_decode over a cache of already rotated keys (no key positions)."""
    torch = _torch()
    i32 = torch.int32
    R, hq, d = q.shape
    nb, hkv, bs, pd = _pool_dims(k_pool, v_pool)
    if pd != d or tuple(out.shape) != (R, hq, d) or out.dtype != q.dtype:
        raise ValueError("q / out / pool head sizes disagree")
    _check_meta("pic_attn_decode_rotated", R, R, d, q_pos, block_table, seq_lens, None, None,
                cos_tab, sin_tab)
    if validation_enabled():
        _validate("pic_attn_decode_rotated", None, q_pos, block_table, seq_lens, None, None, 1,
                  max_seq_len, cos_tab.shape[0], nb)
    _check(_load().pic_attn_decode_rotated(
        _ptr(q, "q"), _ptr(q_pos, "q_pos", i32), _ptr(k_pool, "k_pool", q.dtype),
        _ptr(v_pool, "v_pool", q.dtype), _ptr(block_table, "block_table", i32),
        block_table.shape[1], _ptr(seq_lens, "seq_lens", i32),
        _ptr(cos_tab, "cos_tab", torch.float32), _ptr(sin_tab, "sin_tab", torch.float32),
        cos_tab.shape[0], R, hq, hkv, d, bs, nb, int(max_seq_len), _dtype_code(q),
        _ptr(out, "out"), _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), "pic_attn_decode_rotated")


def pic_attn_prefill_rotated(q, cu_seqlens_q, q_pos, k_pool, v_pool, block_table, seq_lens,
                             cos_tab, sin_tab, max_q_len, max_seq_len, out, workspace,
                             stream=None):
    """pic_attn_prefill over a cache of already rotated keys (no key positions)."""
    torch = _torch()
    i32 = torch.int32
    total_q, hq, d = q.shape
    R = seq_lens.shape[0]
    nb, hkv, bs, pd = _pool_dims(k_pool, v_pool)
    if pd != d or tuple(out.shape) != (total_q, hq, d) or out.dtype != q.dtype:
        raise ValueError("q / out / pool head sizes disagree")
    _check_meta("pic_attn_prefill_rotated", R, total_q, d, q_pos, block_table, seq_lens, None,
                None, cos_tab, sin_tab, cu_seqlens_q)
    if validation_enabled():
        _validate("pic_attn_prefill_rotated", cu_seqlens_q, q_pos, block_table, seq_lens, None,
                  None, int(max_q_len), max_seq_len, cos_tab.shape[0], nb)
    _check(_load().pic_attn_prefill_rotated(
        _ptr(q, "q"), _ptr(cu_seqlens_q, "cu_seqlens_q", i32), _ptr(q_pos, "q_pos", i32),
        _ptr(k_pool, "k_pool", q.dtype), _ptr(v_pool, "v_pool", q.dtype),
        _ptr(block_table, "block_table", i32), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", i32), _ptr(cos_tab, "cos_tab", torch.float32),
        _ptr(sin_tab, "sin_tab", torch.float32), cos_tab.shape[0], R, total_q, int(max_q_len),
        hq, hkv, d, bs, nb, int(max_seq_len), _dtype_code(q), _ptr(out, "out"),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), "pic_attn_prefill_rotated")


def pic_validate_metadata(cu_seqlens_q, q_pos, block_table, seq_lens, cu_seqlens_k, k_pos,
                          max_seq_len, max_pos, num_blocks, block_size=BLOCK_SIZE):
    """Check the device-value preconditions on host (numpy int32) copies.

    Returns (status, message).  cu_seqlens_q may be None for a decode batch.
    """
    arrs = {}
    for name, a in [("cu_seqlens_q", cu_seqlens_q), ("q_pos", q_pos), ("block_table", block_table),
                    ("seq_lens", seq_lens), ("cu_seqlens_k", cu_seqlens_k), ("k_pos", k_pos)]:
        arrs[name] = None if a is None else np.ascontiguousarray(a, dtype=np.int32)
    R = arrs["seq_lens"].shape[0]
    bt = arrs["block_table"]
    stride = bt.shape[1] if bt.ndim == 2 else 0
    total_q = R if arrs["cu_seqlens_q"] is None else int(arrs["q_pos"].shape[0])

    def p(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    buf = ctypes.create_string_buffer(256)
    st = _load().pic_validate_metadata(p(arrs["cu_seqlens_q"]), p(arrs["q_pos"]), p(bt), stride,
                                       p(arrs["seq_lens"]), p(arrs["cu_seqlens_k"]),
                                       p(arrs["k_pos"]), R, total_q, int(max_seq_len),
                                       int(max_pos), int(num_blocks), int(block_size), buf, 256)
    return st, buf.value.decode()


def pic_blocks_copy(src_k_pool, src_v_pool, src_blocks, dst_k_pool, dst_v_pool, dst_blocks,
                    stream=None):
    """Copy whole blocks src_blocks[i] -> dst_blocks[i] between two pools (device or pinned
    host tensors); the id arrays are int32 tensors the device can read."""
    torch = _torch()
    nsb, hkv, bs, d = _pool_dims(src_k_pool, src_v_pool)
    ndb, dhkv, dbs, dd = _pool_dims(dst_k_pool, dst_v_pool)
    if (hkv, bs, d) != (dhkv, dbs, dd) or src_k_pool.dtype != dst_k_pool.dtype:
        raise ValueError("source and destination pools must have the same block shape and dtype")
    if src_blocks.shape != dst_blocks.shape or src_blocks.dim() != 1:
        raise ValueError("src_blocks and dst_blocks must both be [num_pairs]")
    for t, name in [(src_k_pool, "src_k_pool"), (src_v_pool, "src_v_pool"),
                    (dst_k_pool, "dst_k_pool"), (dst_v_pool, "dst_v_pool"),
                    (src_blocks, "src_blocks"), (dst_blocks, "dst_blocks")]:
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be device memory or pinned host memory")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if src_blocks.dtype != torch.int32 or dst_blocks.dtype != torch.int32:
        raise TypeError("block id arrays must be int32")
    _check(_load().pic_blocks_copy(
        src_k_pool.data_ptr(), src_v_pool.data_ptr(), src_blocks.data_ptr(), nsb,
        dst_k_pool.data_ptr(), dst_v_pool.data_ptr(), dst_blocks.data_ptr(), ndb,
        src_blocks.shape[0], hkv, d, _dtype_code(src_k_pool), bs, _stream(stream)),
        "pic_blocks_copy")


def _host_i32(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.int32:
        raise TypeError(f"{name} must be int32")
    return a


def pic_block_hashes(tokens, block_size: int, ssep_token: int = -1, pdep_token: int = -1,
                     seed: int = 0) -> np.ndarray:
    """Span-aware hashes of the full blocks of one host int32 token sequence (uint64)."""
    tok = _host_i32(tokens, "tokens")
    out = np.zeros(max(tok.shape[0] // max(block_size, 1), 1), np.uint64)
    n = _load().pic_block_hashes(tok.ctypes.data, tok.shape[0], block_size, ssep_token,
                                 pdep_token, seed, out.ctypes.data)
    if n < 0:
        _check(n, "pic_block_hashes")
    return out[:n]


def pic_build_block_tables(tokens, cu_seqlens, block_size: int = BLOCK_SIZE,
                           ssep_token: int = -1, pdep_token: int = -1, seed: int = 0,
                           first_block: int = 0, num_blocks: int = 1 << 30, stride=None):
    """Block tables, positions and slot mapping of a batch of host prompts (see pic.h)."""
    tok = _host_i32(tokens, "tokens")
    cu = _host_i32(cu_seqlens, "cu_seqlens")
    R = cu.shape[0] - 1
    lens = np.diff(cu)
    if stride is None:
        stride = max(int(((lens + block_size - 1) // block_size).max()) if R else 1, 1)
    bt = np.zeros((max(R, 1), stride), np.int32)
    total = int(cu[-1]) if R else 0
    k_pos = np.zeros(max(total, 1), np.int32)
    slots = np.zeros(max(total, 1), np.int32)
    hashes = np.zeros(max(int((lens // block_size).sum()) if R else 0, 1), np.uint64)
    nnew = ctypes.c_int(0)
    _check(_load().pic_build_block_tables(
        tok.ctypes.data, cu.ctypes.data, R, block_size, ssep_token, pdep_token, seed,
        first_block, num_blocks, bt.ctypes.data, stride, k_pos.ctypes.data, slots.ctypes.data,
        hashes.ctypes.data, ctypes.byref(nnew)), "pic_build_block_tables")
    nh = int((lens // block_size).sum()) if R else 0
    return dict(block_table=bt[:R], k_pos=k_pos[:total], slot_mapping=slots[:total],
                block_hashes=hashes[:nh], num_new_blocks=int(nnew.value))


def pic_sched_create(policy: int, token_budget: int, max_running: int, num_blocks: int,
                     block_size: int = BLOCK_SIZE) -> int:
    """A scheduler handle (see pic.h: interleaved span-prefill scheduling)."""
    h = ctypes.c_void_p()
    _check(_load().pic_sched_create(policy, token_budget, max_running, num_blocks, block_size,
                                    ctypes.byref(h)), "pic_sched_create")
    return h.value


def pic_sched_destroy(handle) -> None:
    if handle:
        _load().pic_sched_destroy(handle)


def pic_sched_add_span(handle, length: int) -> int:
    sid = _load().pic_sched_add_span(handle, length)
    if sid < 0:
        _check(sid, "pic_sched_add_span")
    return sid


def pic_sched_add_request(handle, arrival_step: int, span_ids, prompt_len: int,
                          output_len: int) -> int:
    ids = _host_i32(np.asarray(span_ids, dtype=np.int32).reshape(-1), "span_ids")
    rid = _load().pic_sched_add_request(handle, arrival_step, ids.ctypes.data if ids.size else None,
                                        ids.shape[0], prompt_len, output_len)
    if rid < 0:
        _check(rid, "pic_sched_add_request")
    return rid


def pic_sched_step(handle, max_seqs: int, max_rows: int, max_keys: int, block_table_stride: int):
    """The next step's batch as a dict of host int32 arrays, or None when every request is done."""
    a = dict(cu_seqlens_q=np.zeros(max_seqs + 1, np.int32), q_pos=np.zeros(max_rows, np.int32),
             slot_mapping=np.zeros(max_rows, np.int32), seq_lens=np.zeros(max_seqs, np.int32),
             cu_seqlens_k=np.zeros(max_seqs + 1, np.int32), k_pos=np.zeros(max_keys, np.int32),
             block_table=np.zeros((max_seqs, block_table_stride), np.int32),
             seq_kind=np.zeros(max_seqs, np.int32), seq_id=np.zeros(max_seqs, np.int32),
             q_begin=np.zeros(max_seqs, np.int32))
    b = _SchedBatch(max_seqs=max_seqs, max_rows=max_rows, max_keys=max_keys,
                    block_table_stride=block_table_stride,
                    **{k: v.ctypes.data for k, v in a.items()})
    st = _load().pic_sched_step(handle, ctypes.byref(b))
    if st < 0:
        _check(st, "pic_sched_step")
    if st == 0:
        return None
    n, tq, tk = b.num_seqs, b.total_q, b.total_keys
    return dict(step=b.step, num_seqs=n, total_q=tq, max_q_len=b.max_q_len,
                max_seq_len=b.max_seq_len, total_keys=tk, num_finished=b.num_finished,
                cu_seqlens_q=a["cu_seqlens_q"][:n + 1], q_pos=a["q_pos"][:tq],
                slot_mapping=a["slot_mapping"][:tq], seq_lens=a["seq_lens"][:n],
                cu_seqlens_k=a["cu_seqlens_k"][:n + 1], k_pos=a["k_pos"][:tk],
                block_table=a["block_table"][:n], seq_kind=a["seq_kind"][:n],
                seq_id=a["seq_id"][:n], q_begin=a["q_begin"][:n])


class Scheduler:
    """Owns a pic_sched handle: spans and requests are added, then steps drawn until None."""

    def __init__(self, policy: int, token_budget: int, max_running: int, num_blocks: int,
                 max_seqs: int, max_keys: int, block_table_stride: int):
        self.handle = pic_sched_create(policy, token_budget, max_running, num_blocks)
        self.caps = (max_seqs, token_budget, max_keys, block_table_stride)

    def add_span(self, length: int) -> int:
        return pic_sched_add_span(self.handle, length)

    def add_request(self, arrival_step: int, span_ids, prompt_len: int, output_len: int) -> int:
        return pic_sched_add_request(self.handle, arrival_step, span_ids, prompt_len, output_len)

    def step(self):
        return pic_sched_step(self.handle, *self.caps)

    def close(self):
        pic_sched_destroy(self.handle)
        self.handle = None

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            self.close()


def pic_decode_num_splits(seq_len: int, dtype: int = PIC_BF16) -> int:
    return int(_load().pic_decode_num_splits(seq_len, dtype))


def pic_decode_split_len(seq_len: int, dtype: int = PIC_BF16) -> int:
    return int(_load().pic_decode_split_len(seq_len, dtype))


def pic_decode_chunk_start(seq_len: int, chunk: int, dtype: int = PIC_BF16) -> int:
    return int(_load().pic_decode_chunk_start(seq_len, chunk, dtype))


def pic_stream_read(src, workgroups: int, sink, order=None, piece_bytes: int = 0,
                    stream=None) -> None:
    """Measurement helper: read the device tensor `src` once with a plain streaming kernel
    of `workgroups` x 256 lanes, front to back, or as pieces of piece_bytes in the order of
    the int32 device tensor `order`; sink: a device tensor of >= workgroups * 256 int32."""
    torch = _torch()
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < workgroups * 256 * 4:
        raise ValueError("sink must hold workgroups * 256 uint32")
    if order is not None and (piece_bytes <= 0 or order.numel() * piece_bytes != nbytes):
        raise ValueError("order must list nbytes / piece_bytes pieces")
    _check(_load().pic_stream_read(_ptr(src, "src"), nbytes,
                                   _ptr(order, "order", torch.int32) if order is not None else None,
                                   int(piece_bytes), int(workgroups), _ptr(sink, "sink"),
                                   _stream(stream)), "pic_stream_read")


class TimingEvent:
    """A HIP event for timing only (pic_timing_event_create: no system-scope fence at its
    records).  record(stream=None) and elapsed_time(end) in ms, as torch.cuda.Event."""

    def __init__(self):
        lib = _load()
        h = ctypes.c_void_p()
        _check(lib.pic_timing_event_create(ctypes.byref(h)), "pic_timing_event_create")
        self.handle = h.value

    def record(self, stream=None):
        _check(_load().pic_timing_event_record(ctypes.c_void_p(self.handle), _stream(stream)),
               "pic_timing_event_record")

    def elapsed_time(self, end) -> float:
        ms = ctypes.c_float()
        _check(_load().pic_timing_event_elapsed_ms(ctypes.c_void_p(self.handle),
                                                   ctypes.c_void_p(end.handle),
                                                   ctypes.byref(ms)),
               "pic_timing_event_elapsed_ms")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.pic_timing_event_destroy(ctypes.c_void_p(self.handle))
            self.handle = None


def pic_set_kernel_events(before=None, after=None) -> None:
    """Have the main kernel of every following attention call on this thread record two
    events at its start and end (None, None turns it off); elapsed_time(before, after) is
    then that kernel's duration alone.  The events are TimingEvent objects or
    torch.cuda.Event objects (a torch event whose HIP event does not exist yet is recorded
    once here)."""
    lib = _load()
    if (before is None) != (after is None):
        raise ValueError("pass both events or neither")
    if before is None:
        _check(lib.pic_set_kernel_events(None, None), "pic_set_kernel_events")
        return
    handles = []
    for e in (before, after):
        if isinstance(e, TimingEvent):
            handles.append(e.handle)
        else:
            if not e.cuda_event:
                e.record()
            handles.append(e.cuda_event)
    _check(lib.pic_set_kernel_events(ctypes.c_void_p(handles[0]), ctypes.c_void_p(handles[1])),
           "pic_set_kernel_events")

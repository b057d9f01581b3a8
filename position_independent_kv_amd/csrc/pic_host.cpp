// Host-side part of libpic: status strings, argument checks, workspace
// sizing, split policy and the metadata validator.  No HIP calls here, so the
// same file also builds with g++ alone (the CPU tests run it under
// AddressSanitizer / UndefinedBehaviorSanitizer).
#include <stdio.h>
#include <string.h>

#include "pic.h"
#include "pic_common.hpp"
#include "pic_host.hpp"

extern "C" const char* pic_status_string(int status) {
  switch (status) {
    case PIC_OK: return "PIC_OK";
    case PIC_EINVAL: return "PIC_EINVAL: invalid argument";
    case PIC_EUNSUPPORTED: return "PIC_EUNSUPPORTED: unsupported shape or dtype";
    case PIC_EWORKSPACE: return "PIC_EWORKSPACE: workspace missing or too small";
    case PIC_EHIP: return "PIC_EHIP: HIP launch failed";
    default: return "unknown pic_status";
  }
}

extern "C" int pic_version(void) { return 100; }

extern "C" int pic_decode_num_splits(int seq_len, int dtype) {
  return pic::num_splits(seq_len, pic::kstep_for(dtype));
}

extern "C" int pic_decode_split_len(int seq_len, int dtype) {
  return pic::split_len(seq_len, pic::kstep_for(dtype));
}

extern "C" int pic_decode_chunk_start(int seq_len, int chunk, int dtype) {
  const int S = pic::num_splits(seq_len, pic::kstep_for(dtype));
  if (chunk < 0 || chunk > S) return -1;
  return pic::chunk_start(seq_len, chunk, pic::kstep_for(dtype));
}

namespace pic {

int check_dtype_dims(int dtype, int head_dim, int block_size) {
  if (dtype != PIC_F32 && dtype != PIC_BF16) return PIC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PIC_EUNSUPPORTED;
  if (block_size != kBlockSize) return PIC_EUNSUPPORTED;
  return PIC_OK;
}

int check_heads(int hq, int hkv) {
  if (hq <= 0 || hkv <= 0) return PIC_EINVAL;
  if (hq % hkv) return PIC_EUNSUPPORTED;
  const int g = hq / hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return PIC_EUNSUPPORTED;
  return PIC_OK;
}

int check_attn_common(const AttnHostArgs& a, bool key_positions, bool decode) {
  if (a.num_reqs < 0 || a.total_q < 0 || a.max_seq_len < 0 || a.hq <= 0 || a.hkv <= 0)
    return check_attn_args(a, key_positions, 0);
  const WorkspaceLayout w = workspace_layout(a.num_reqs, a.total_q, a.max_seq_len, a.hq, a.hkv,
                                             a.head_dim, decode);
  return check_attn_args(a, key_positions, w.total);
}

int check_attn_args(const AttnHostArgs& a, bool key_positions, size_t need) {
  if (a.num_reqs < 0 || a.total_q < 0 || a.max_seq_len < 0 || a.num_blocks < 0 ||
      a.block_table_stride < 0 || a.max_pos <= 0)
    return PIC_EINVAL;
  int st = check_dtype_dims(a.dtype, a.head_dim, a.block_size);
  if (st) return st;
  st = check_heads(a.hq, a.hkv);
  if (st) return st;
  if (a.num_reqs == 0 || a.total_q == 0) return PIC_OK;
  if (!a.q || !a.q_pos || !a.k_pool || !a.v_pool || !a.block_table || !a.seq_lens ||
      !a.cos_tab || !a.sin_tab || !a.out)
    return PIC_EINVAL;
  if (key_positions && (!a.cu_seqlens_k || !a.k_pos)) return PIC_EINVAL;
  if (a.num_blocks == 0 || a.block_table_stride == 0) return PIC_EINVAL;
  if ((long long)a.block_table_stride * a.block_size < a.max_seq_len) return PIC_EINVAL;
  if (!a.workspace) return PIC_EWORKSPACE;
  if (a.workspace_bytes < need) return PIC_EWORKSPACE;
  return PIC_OK;
}

}  // namespace pic

extern "C" size_t pic_attn_workspace_size(int num_reqs, int total_q, int max_seq_len,
                                          int num_q_heads, int num_kv_heads, int head_dim,
                                          int dtype) {
  if (num_reqs < 0 || total_q < 0 || max_seq_len < 0) return 0;
  if (pic::check_dtype_dims(dtype, head_dim, pic::kBlockSize)) return 0;
  if (pic::check_heads(num_q_heads, num_kv_heads)) return 0;
  return pic::workspace_layout(num_reqs, total_q, max_seq_len, num_q_heads, num_kv_heads,
                               head_dim).total;
}

extern "C" size_t pic_attn_decode_shared_workspace_size(int num_reqs, int max_seq_len,
                                                        int num_q_heads, int num_kv_heads,
                                                        int head_dim, int dtype) {
  if (num_reqs < 0 || max_seq_len < 0) return 0;
  if (pic::check_dtype_dims(dtype, head_dim, pic::kBlockSize)) return 0;
  if (pic::check_heads(num_q_heads, num_kv_heads)) return 0;
  const pic::SharedDecodeLayout w =
      pic::shared_decode_layout(num_reqs, max_seq_len, num_q_heads, num_kv_heads, head_dim);
  return w.supported ? w.total : 0;
}

static int fail(char* msg, int msg_len, const char* fmt, long long a, long long b) {
  if (msg && msg_len > 0) snprintf(msg, (size_t)msg_len, fmt, a, b);
  return PIC_EINVAL;
}

extern "C" int pic_validate_metadata(const int32_t* cu_q, const int32_t* q_pos,
                                     const int32_t* block_table, int stride,
                                     const int32_t* seq_lens, const int32_t* cu_k,
                                     const int32_t* k_pos, int num_reqs, int total_q,
                                     int max_seq_len, int max_pos, int num_blocks,
                                     int block_size, char* msg, int msg_len) {
  if (msg && msg_len > 0) msg[0] = 0;
  if (num_reqs < 0 || total_q < 0 || block_size <= 0 || stride < 0)
    return fail(msg, msg_len, "bad sizes (num_reqs %lld, total_q %lld)", num_reqs, total_q);
  if (num_reqs == 0) return PIC_OK;
  if (!q_pos || !block_table || !seq_lens || !cu_k || !k_pos)
    return fail(msg, msg_len, "null array (%lld, %lld)", 0, 0);
  if (!cu_q && total_q != num_reqs)
    return fail(msg, msg_len, "decode batch needs total_q == num_reqs (%lld vs %lld)", total_q,
                num_reqs);
  if (cu_q && (cu_q[0] != 0 || cu_q[num_reqs] != total_q))
    return fail(msg, msg_len, "cu_seqlens_q must run from 0 to total_q (%lld, %lld)", cu_q[0],
                cu_q[num_reqs]);
  if (cu_k[0] != 0) return fail(msg, msg_len, "cu_seqlens_k[0] = %lld, want 0%lld", cu_k[0], 0);
  for (int r = 0; r < num_reqs; ++r) {
    const long long L = seq_lens[r];
    const long long q0 = cu_q ? cu_q[r] : r;
    const long long ql = cu_q ? (long long)cu_q[r + 1] - cu_q[r] : 1;
    if (ql < 0) return fail(msg, msg_len, "request %lld: negative q_len %lld", r, ql);
    if (L < 0 || L > max_seq_len)
      return fail(msg, msg_len, "request %lld: seq_len %lld outside [0, max_seq_len]", r, L);
    if (ql > L) return fail(msg, msg_len, "request %lld: q_len > seq_len (%lld)", r, ql);
    if ((long long)cu_k[r + 1] - cu_k[r] != L)
      return fail(msg, msg_len, "request %lld: cu_seqlens_k step %lld != seq_len", r,
                  (long long)cu_k[r + 1] - cu_k[r]);
    const long long nb = (L + block_size - 1) / block_size;
    if (nb > stride) return fail(msg, msg_len, "request %lld needs %lld blocks > stride", r, nb);
    for (long long b = 0; b < nb; ++b) {
      const long long id = block_table[(long long)r * stride + b];
      if (id < 0 || id >= num_blocks)
        return fail(msg, msg_len, "request %lld: block id %lld out of range", r, id);
    }
    for (long long j = 0; j < L; ++j) {
      const long long p = k_pos[cu_k[r] + j];
      if (p < 0 || p >= max_pos)
        return fail(msg, msg_len, "request %lld: key position %lld out of range", r, p);
    }
    for (long long i = 0; i < ql; ++i) {
      const long long p = q_pos[q0 + i];
      if (p < 0 || p >= max_pos)
        return fail(msg, msg_len, "request %lld: query position %lld out of range", r, p);
    }
  }
  return PIC_OK;
}

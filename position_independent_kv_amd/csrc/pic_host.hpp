// Host-side helpers shared by the entry points (plain C++, no HIP).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pic {

struct AttnHostArgs {
  const void* q;
  const int32_t* cu_seqlens_q;
  const int32_t* q_pos;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  int block_table_stride;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_k;
  const int32_t* k_pos;
  const float* cos_tab;
  const float* sin_tab;
  int max_pos;
  int num_reqs;
  int total_q;
  int max_q_len;
  int hq;
  int hkv;
  int head_dim;
  int block_size;
  int num_blocks;
  int max_seq_len;
  int dtype;
  void* out;
  void* workspace;
  size_t workspace_bytes;
  // decode with append: request r's new token, [num_reqs][hkv][head_dim]
  const void* new_k = nullptr;
  const void* new_v = nullptr;
};

int check_dtype_dims(int dtype, int head_dim, int block_size);
int check_heads(int hq, int hkv);
// Host-visible argument checks of an attention call; key_positions: the call
// reads cu_seqlens_k and k_pos (the position-free kernels do); decode: a
// pic_attn_decode call, whose workspace has no prefill-split regions.
int check_attn_common(const AttnHostArgs& a, bool key_positions, bool decode);
// The same checks against a workspace requirement of `need` bytes.
int check_attn_args(const AttnHostArgs& a, bool key_positions, size_t need);

}  // namespace pic

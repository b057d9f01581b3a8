// Shared constants and pure functions of the library (host code and kernels).
// Plain C++: this header is also compiled by the host-only build that the
// CPU tests run under sanitizers.  constexpr functions are usable from both
// host and device code under hipcc.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pic {

constexpr int kBlockSize = 16;      // tokens per KV block
constexpr int kWaves = 4;           // waves (of 64 lanes) per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kPrefillRows = 128;   // query rows (tokens x group heads) per prefill tile
constexpr int kSplitTarget = 384;   // target keys per decode chunk (one workgroup)
constexpr int kMaxGroup = 16;       // q heads per kv head held in one MFMA column tile

// Keys consumed per inner step: two 16-key MFMA tiles for bf16, one for fp32.
constexpr int kstep_for(int dtype) { return dtype == 1 ? 32 : 16; }

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Key chunks of a request with L keys: round(L / kSplitTarget) chunks (at
// least one), of equal length rounded up to whole inner steps, so chunks stay
// within [0.67, 1.5] x the target.  A pure function of L: a request is split
// the same way in any batch, so its result does not depend on the batch.
constexpr int num_chunks_target(int L) {
  return L <= 0 ? 1 : ((L + kSplitTarget / 2) / kSplitTarget > 0 ? (L + kSplitTarget / 2) / kSplitTarget : 1);
}
constexpr int split_len(int L, int kstep) {
  return L <= 0 ? kstep : cdiv(cdiv(L, num_chunks_target(L)), kstep) * kstep;
}
constexpr int num_splits(int L, int kstep) { return L <= 0 ? 1 : cdiv(L, split_len(L, kstep)); }
// Upper bound of num_splits over all L <= max_len.
constexpr int max_splits(int max_len) { return max_len <= 0 ? 1 : cdiv(max_len, kSplitTarget) + 1; }

// Work-list item kinds (the mixed launch).
constexpr int kItemPrefill = 0;
constexpr int kItemDecode = 1;

// Byte layout of the attention workspace.
struct WorkspaceLayout {
  size_t count_off;     // int: number of work items written by the planner
  size_t items_off;     // int4[max_items]: work list
  size_t ml_off;        // float2[num_reqs * hkv * s_max * group]: (max, sum) per chunk
  size_t o_off;         // float[num_reqs * hkv * s_max * group * head_dim]: chunk outputs
  size_t total;
  int s_max;            // chunks per request, upper bound
  int nhg;              // kv-head groups of kWaves heads (an upper bound for wider groups)
  long long max_items;  // work-list capacity
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline WorkspaceLayout workspace_layout(int num_reqs, int total_q, int max_seq_len, int hq,
                                        int hkv, int head_dim) {
  WorkspaceLayout w{};
  const int group = hq / hkv;
  w.s_max = max_splits(max_seq_len);
  w.nhg = cdiv(hkv, kWaves);
  // prefill tiles: sum_r ceil(q_len_r * group / rows) <= total_q*group/rows + num_reqs
  const long long tiles = (long long)hkv * ((long long)total_q * group / kPrefillRows + num_reqs);
  const long long dec = (long long)num_reqs * w.s_max * w.nhg;
  w.max_items = tiles + dec;
  size_t off = 0;
  w.count_off = off;
  off = align_up(off + 16, 256);
  w.items_off = off;
  off = align_up(off + (size_t)w.max_items * 16, 256);
  const size_t parts = (size_t)num_reqs * hkv * w.s_max * group;
  w.ml_off = off;
  off = align_up(off + parts * 8, 256);
  w.o_off = off;
  off = align_up(off + parts * head_dim * 4, 256);
  w.total = off;
  return w;
}

}  // namespace pic

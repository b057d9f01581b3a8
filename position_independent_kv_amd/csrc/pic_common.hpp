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
constexpr int kPrefillRows = 128;   // query rows (tokens x group heads) per fp32 prefill tile
// Target keys per decode chunk (one workgroup).  Measured against 384, 640 and 768
// on MI355X with every call cold, over decode batches of 32-128 requests x 2k-8k keys:
// 512 was fastest on 14 of 18 batches (geometric mean -4% against 384).
constexpr int kSplitTarget = 512;
constexpr int kMaxGroup = 16;       // q heads per kv head held in one MFMA column tile

// Keys consumed per inner step: two 16-key MFMA tiles for bf16, one for fp32.
constexpr int kstep_for(int dtype) { return dtype == 1 ? 32 : 16; }

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Key chunks of a request with L keys: S = round(L / kSplitTarget) chunks (at
// least one, at most one per inner step), the n = cdiv(L, kstep) inner steps
// dealt out evenly: chunk s covers steps [s n / S, (s + 1) n / S), so no chunk
// is more than one step longer than another and all stay within about
// [0.67, 1.5] x the target.  (Equal chunks rounded up to whole steps left a
// short last chunk, and the mixed launch, which deals its decode chunks to the
// XCDs chunk level by chunk level, gave all of a batch's short chunks to one
// XCD.)  A pure function of L: a request is split the same way in any batch,
// so its result does not depend on the batch.
constexpr int num_chunks_target(int L) {
  return L <= 0 ? 1 : ((L + kSplitTarget / 2) / kSplitTarget > 0 ? (L + kSplitTarget / 2) / kSplitTarget : 1);
}
constexpr int num_splits(int L, int kstep) {
  return L <= 0 ? 1 : (num_chunks_target(L) < cdiv(L, kstep) ? num_chunks_target(L) : cdiv(L, kstep));
}
// First key of chunk s (chunk num_splits(L) starts at L).
constexpr int chunk_start(int L, int s, int kstep) {
  return L <= 0 ? 0
                : ((long long)s * cdiv(L, kstep) / num_splits(L, kstep) * kstep < L
                       ? (int)((long long)s * cdiv(L, kstep) / num_splits(L, kstep) * kstep)
                       : L);
}
// Key slots of the longest chunk (whole inner steps).
constexpr int split_len(int L, int kstep) {
  return L <= 0 ? kstep : cdiv(cdiv(L, kstep), num_splits(L, kstep)) * kstep;
}
// Upper bound of num_splits over all L <= max_len, and the exact maximum:
// num_splits(L) <= num_chunks_target(L) (chunks are at least L / target long),
// which never decreases with L.  The decode grid is sized by it, so a batch
// of equal contexts launches no empty chunk workgroups.
constexpr int max_splits(int max_len) { return num_chunks_target(max_len); }

// Work-list item kinds (the mixed launch).
constexpr int kItemPrefill = 0;
constexpr int kItemDecode = 1;

// Key splitting of bf16 prefill tiles (the mixed launch).  A launch whose
// prefill tiles are fewer than kSplitCUs (the compute units to fill) splits
// the key range of each tile of a request with L keys into
// min(kSplitCUs / tiles, L / kPrefillChunkMin) chunks, each a work item that
// writes a partial result; a merge kernel combines them.  The decision
// depends on the launch's total prefill tiles, so a request's prefill rows
// are bit-identical between launches that split it the same way (always
// when the launch has kSplitCUs tiles or more, or the request has fewer than
// 2 * kPrefillChunkMin keys).  Split items of one launch never exceed
// kSplitCUs, nor split tiles kSplitCUs / 2.
constexpr int kSplitCUs = 256;
constexpr int kPrefillChunkMin = 1024;
constexpr int kPrefillTileRows = 256;  // query rows of one bf16 prefill tile (8 waves x 32)

// Whether a mixed launch of this size might split prefill tiles: a lower
// bound of its prefill tiles, from the rows that are not decode rows, is
// below kSplitCUs, and some context is at least two chunks long.
constexpr bool prefill_split_possible(long long total_q, long long num_reqs, int hq, int hkv,
                                      long long max_seq_len) {
  return hkv > 0 && max_seq_len >= 2LL * kPrefillChunkMin &&
         (long long)hkv * ((total_q - num_reqs > 0 ? total_q - num_reqs : 0) * (hq / hkv) /
                           kPrefillTileRows) < kSplitCUs;
}

// Byte layout of the attention workspace.
struct WorkspaceLayout {
  size_t count_off;     // int[2]: work items written by the planner; 1 if it refused an
                        // overflowing work list (the mixed launch then writes NaN)
  size_t items_off;     // int4[max_items]: work list
  size_t ml_off;        // float2[num_reqs * hkv * s_max * group]: (max, sum) per chunk
  size_t o_off;         // float[num_reqs * hkv * s_max * group * head_dim]: chunk outputs
  size_t pf_count_off;  // int: split prefill tiles written by the planner
  size_t pf_tiles_off;  // int4[kSplitCUs / 2]: (request, kv head, tile, first item) per split tile
  size_t pf_ml_off;     // float2[kSplitCUs][kPrefillTileRows]: (max, sum) per split item row
  size_t pf_o_off;      // float[kSplitCUs][kPrefillTileRows][head_dim]: split item outputs
  bool pf_split;        // prefill tiles may be split (the four regions above exist)
  size_t total;
  int s_max;            // chunks per request, upper bound
  int nhg;              // kv-head groups of kWaves heads (an upper bound for wider groups)
  long long max_items;  // work-list capacity
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// decode: the layout of a pic_attn_decode call, which never splits prefill
// tiles (the same offsets, without the split regions at the end).
inline WorkspaceLayout workspace_layout(int num_reqs, int total_q, int max_seq_len, int hq,
                                        int hkv, int head_dim, bool decode = false) {
  WorkspaceLayout w{};
  const int group = hq / hkv;
  w.s_max = max_splits(max_seq_len);
  w.nhg = cdiv(hkv, kWaves);
  // prefill tiles: sum_r ceil(q_len_r * group / rows) <= total_q*group/rows + num_reqs
  const long long tiles = (long long)hkv * ((long long)total_q * group / kPrefillRows + num_reqs);
  const long long dec = (long long)num_reqs * w.s_max * w.nhg;
  // a launch that splits prefill tiles has at most kSplitCUs prefill items
  w.max_items = tiles + dec +
                (prefill_split_possible(total_q, num_reqs, hq, hkv, max_seq_len) ? kSplitCUs : 0);
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
  w.pf_split = !decode && prefill_split_possible(total_q, num_reqs, hq, hkv, max_seq_len);
  w.pf_count_off = w.pf_tiles_off = w.pf_ml_off = w.pf_o_off = off;
  if (w.pf_split) {
    w.pf_count_off = off;
    off = align_up(off + 16, 256);
    w.pf_tiles_off = off;
    off = align_up(off + (size_t)(kSplitCUs / 2) * 16, 256);
    w.pf_ml_off = off;
    off = align_up(off + (size_t)kSplitCUs * kPrefillTileRows * 8, 256);
    w.pf_o_off = off;
    off = align_up(off + (size_t)kSplitCUs * kPrefillTileRows * head_dim * 4, 256);
  }
  w.total = off;
  return w;
}

// Shared-span decode (pic_attn_decode_shared): a request's chunk boundaries
// are decided by its blocks' physical ids, so two requests that hold the same
// span at different offsets cut it at the same blocks and compute identical
// chunks, which the planner then runs side by side on one XCD.
constexpr int kCdcCandMask = 15;      // a block is a cut candidate with probability 1/16
constexpr int kCdcMinGap = 12;        // blocks between two cuts, at least
constexpr int kCdcMaxGap = 38;        // a longer gap between cuts is split ...
constexpr int kCdcSplitGap = 24;      // ... into cdiv(gap, 24) equal parts
constexpr int kCdcMaxBlocks = 65536;  // blocks of one request the planner handles
constexpr int kCdcSortMax = 8192;     // chunks the ordering kernel groups (more: request order)
constexpr int kCdcPosBuckets = 8192;  // start-block classes of chunks that occur once

// Byte layout of the shared-span decode's workspace.
struct SharedDecodeLayout {
  size_t count_off;     // int: work items written by the planner
  size_t items_off;     // int4[max_items]: work list
  size_t ml_off;        // float2[num_reqs * hkv * s_max * group]: (max, sum) per chunk
  size_t o_off;         // float[... * head_dim]: chunk outputs
  size_t cnt_off;       // int[num_reqs]: chunks per request
  size_t start_off;     // int[num_reqs][s_max + 1]: chunk start blocks, then the block count
  size_t coff_off;      // int[num_reqs + 1]: first chunk of each request in the list
  size_t total;
  int s_max;            // chunks per request, upper bound
  int nhg;              // kv-head groups of kWaves heads
  long long max_items;  // work-list capacity
  bool supported;       // within the planner's limits
};

// Chunks are at least kCdcMinGap blocks long except the first and the last,
// so a request of nb blocks has at most nb / kCdcMinGap + 3 of them.
inline SharedDecodeLayout shared_decode_layout(int num_reqs, int max_seq_len, int hq, int hkv,
                                               int head_dim) {
  SharedDecodeLayout w{};
  const int group = hq / hkv;
  const int nb_max = cdiv(max_seq_len > 0 ? max_seq_len : 0, kBlockSize);
  w.s_max = cdiv(nb_max, kCdcMinGap) + 3;
  w.nhg = cdiv(hkv, kWaves);
  w.max_items = (long long)num_reqs * w.s_max * w.nhg;
  w.supported = nb_max <= kCdcMaxBlocks && w.max_items <= 0x7fffffffLL &&
                (long long)num_reqs * hkv <= 0x7fffffffLL;
  const size_t parts = (size_t)num_reqs * hkv * w.s_max * group;
  size_t off = 0;
  w.count_off = off;
  off = align_up(off + 16, 256);
  w.items_off = off;
  off = align_up(off + (size_t)w.max_items * 16, 256);
  w.ml_off = off;
  off = align_up(off + parts * 8, 256);
  w.o_off = off;
  off = align_up(off + parts * head_dim * 4, 256);
  w.cnt_off = off;
  off = align_up(off + (size_t)num_reqs * 4, 256);
  w.start_off = off;
  off = align_up(off + (size_t)num_reqs * (w.s_max + 1) * 4, 256);
  w.coff_off = off;
  off = align_up(off + ((size_t)num_reqs + 1) * 4, 256);
  w.total = off;
  return w;
}

}  // namespace pic

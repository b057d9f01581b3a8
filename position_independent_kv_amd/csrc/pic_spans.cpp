// Span-aware block hashing and block-table construction (host code).
//
// MiniPIC §2.2 (user-controlled cache-reuse primitives): spans are padded to
// KV-block boundaries, and two special tokens at the start of a block change
// how that block's prefix-cache hash is chained:
//   - default:           h_i = H(h_{i-1}, x_i)   (the hash of block i covers
//                        its whole prefix, through the chain);
//   - SSEP block start:  h_i = H(h_0, x_i)       (the chain restarts, so a
//                        span hashes the same whatever precedes it);
//   - PDEP block start:  h_i = H(h_0, x_{<=i})   (the hash covers every
//                        token of the prompt up to and including block i,
//                        across earlier SSEP restarts).
// x_i is the token ids of block i and h_0 the caller's seed.  H is FNV-1a
// 64 (Fowler/Noll/Vo) over the little-endian bytes of its arguments: the
// 8-byte parent hash, then each token id as 4 bytes.  Only full blocks are
// hashed; a trailing partial block never matches another.
#include <stdint.h>
#include <string.h>

#include <unordered_map>
#include <vector>

#include "pic.h"
#include "pic_common.hpp"

namespace pic {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

struct Fnv {
  uint64_t h = kFnvOffset;
  void byte(uint8_t b) {
    h ^= b;
    h *= kFnvPrime;
  }
  void u64(uint64_t x) {
    for (int i = 0; i < 8; ++i) byte((uint8_t)(x >> (8 * i)));
  }
  void i32(int32_t x) {
    const uint32_t u = (uint32_t)x;
    for (int i = 0; i < 4; ++i) byte((uint8_t)(u >> (8 * i)));
  }
};

// Hashes of the full blocks of one token sequence (see the rules above).
static void hash_blocks(const int32_t* tok, int n, int bs, int32_t ssep, int32_t pdep,
                        uint64_t seed, uint64_t* out) {
  const int nb = n / bs;
  Fnv prompt;  // running H(h_0, x_0 .. ) over the whole prompt, for PDEP blocks
  prompt.u64(seed);
  uint64_t parent = seed;
  for (int b = 0; b < nb; ++b) {
    const int32_t* x = tok + (size_t)b * bs;
    for (int j = 0; j < bs; ++j) prompt.i32(x[j]);
    uint64_t h;
    if (pdep >= 0 && x[0] == pdep) {
      h = prompt.h;
    } else {
      Fnv f;
      f.u64((ssep >= 0 && x[0] == ssep) ? seed : parent);
      for (int j = 0; j < bs; ++j) f.i32(x[j]);
      h = f.h;
    }
    out[b] = h;
    parent = h;
  }
}

}  // namespace pic

extern "C" int pic_block_hashes(const int32_t* tokens, int num_tokens, int block_size,
                                int32_t ssep_token, int32_t pdep_token, uint64_t seed,
                                uint64_t* hashes) {
  if (num_tokens < 0 || block_size <= 0) return PIC_EINVAL;
  if (num_tokens / block_size > 0 && (!tokens || !hashes)) return PIC_EINVAL;
  pic::hash_blocks(tokens, num_tokens, block_size, ssep_token, pdep_token, seed, hashes);
  return num_tokens / block_size;
}

extern "C" int pic_build_block_tables(const int32_t* tokens, const int32_t* cu_seqlens,
                                      int num_reqs, int block_size, int32_t ssep_token,
                                      int32_t pdep_token, uint64_t seed, int first_block,
                                      int num_blocks, int32_t* block_table,
                                      int block_table_stride, int32_t* k_pos,
                                      int32_t* slot_mapping, uint64_t* block_hashes,
                                      int* num_new_blocks) {
  if (num_reqs < 0 || block_size != pic::kBlockSize || first_block < 0 || num_blocks < 0 ||
      block_table_stride < 0)
    return PIC_EINVAL;
  if (num_new_blocks) *num_new_blocks = 0;
  if (num_reqs == 0) return PIC_OK;
  if (!tokens || !cu_seqlens || !block_table || !k_pos || !slot_mapping || !num_new_blocks)
    return PIC_EINVAL;
  if (cu_seqlens[0] != 0) return PIC_EINVAL;
  for (int r = 0; r < num_reqs; ++r) {
    const int len = cu_seqlens[r + 1] - cu_seqlens[r];
    if (len < 0) return PIC_EINVAL;
    if ((long long)(len + block_size - 1) / block_size > block_table_stride) return PIC_EINVAL;
  }
  std::unordered_map<uint64_t, int32_t> seen;  // full-block hash -> physical block
  std::vector<uint64_t> h;
  int next = first_block;
  for (int r = 0; r < num_reqs; ++r) {
    const int t0 = cu_seqlens[r];
    const int len = cu_seqlens[r + 1] - t0;
    const int nfull = len / block_size;
    const int nblk = (len + block_size - 1) / block_size;
    h.assign((size_t)nfull, 0);
    pic::hash_blocks(tokens + t0, len, block_size, ssep_token, pdep_token, seed, h.data());
    int32_t* bt = block_table + (size_t)r * block_table_stride;
    for (int b = 0; b < block_table_stride; ++b) bt[b] = 0;
    for (int b = 0; b < nblk; ++b) {
      int32_t blk;
      bool fresh = true;
      if (b < nfull) {
        auto it = seen.find(h[(size_t)b]);
        if (it != seen.end()) {
          blk = it->second;
          fresh = false;
        } else {
          if (next >= num_blocks) return PIC_EINVAL;  // pool exhausted
          blk = next++;
          seen.emplace(h[(size_t)b], blk);
        }
      } else {  // a partial block is private to its request
        if (next >= num_blocks) return PIC_EINVAL;
        blk = next++;
      }
      bt[b] = blk;
      const int n_in = b < nfull ? block_size : len - b * block_size;
      for (int j = 0; j < n_in; ++j) {
        const int t = b * block_size + j;
        slot_mapping[t0 + t] = fresh ? blk * block_size + j : -1;
      }
    }
    for (int t = 0; t < len; ++t) k_pos[t0 + t] = t;
  }
  if (block_hashes) {
    size_t o = 0;
    for (int r = 0; r < num_reqs; ++r) {
      const int t0 = cu_seqlens[r];
      const int len = cu_seqlens[r + 1] - t0;
      pic::hash_blocks(tokens + t0, len, block_size, ssep_token, pdep_token, seed,
                       block_hashes + o);
      o += (size_t)(len / block_size);
    }
  }
  *num_new_blocks = next - first_block;
  return PIC_OK;
}

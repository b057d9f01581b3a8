// pic_cache_write: store new tokens' keys and values, unrotated, into the pools.
//
// MiniPIC §2.1: the cache holds non-rotated key vectors k~_j, which is what
// lets one physical block serve requests at different offsets without being
// rewritten.  This is a pure scatter: the stored bytes are the input bytes.
//
// K goes to k_pool[block][h][offset][d] (one contiguous row per token and
// head); V goes to v_pool[block][h][d][offset] (transposed inside the block so
// that the attention kernels read runs of consecutive keys as matrix-core
// operands).  One launch writes both.
#include <hip/hip_runtime.h>

#include "pic.h"
#include "pic_common.hpp"

namespace pic {

// One workgroup per (group of 16 consecutive input tokens, kv head); D is the
// head size, T the element type, and each thread moves 16-byte pieces.  K:
// each token's row is one contiguous run in the pool, its pieces in
// neighbouring lanes.  V: when the group's 16 slots are offsets 0..15 of one
// block (a block filled in order, the usual prefill case), the group's rows
// go through LDS and come out transposed as 16-byte runs of the block's V^T
// rows; otherwise every element goes to its own place, the 16 tokens of the
// group in neighbouring lanes, so that tokens in consecutive slots fill one
// V^T row segment per store.  Every load of a thread is issued before its
// stores.  Tokens whose slot is negative or past the pool are skipped.
// (2-byte V loads in the in-order case and token-major V stores otherwise
// ran the 32,896-token mixed batch at 93 us, 2.9 TB/s of reads + writes.)
template <typename T, int D>
__global__ void __launch_bounds__(256) cache_write_kernel(const T* __restrict__ k,
                                                          const T* __restrict__ v,
                                                          const int32_t* __restrict__ slots,
                                                          long long num_tokens, int hkv,
                                                          T* __restrict__ k_pool,
                                                          T* __restrict__ v_pool,
                                                          long long num_slots) {
  constexpr int VEC = 16 / sizeof(T);   // elements per piece
  constexpr int CH = D / VEC;           // pieces per token row
  constexpr int PG = kBlockSize * CH;   // pieces of the group (one head)
  constexpr int UPR = kBlockSize / VEC;  // pieces per V^T row of a block
  constexpr int NP = (PG + 255) / 256;  // pieces per thread
  static_assert(PG % 64 == 0, "whole waves of pieces");
  __shared__ __attribute__((aligned(16))) T vs[kBlockSize * D];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const long long groups = (num_tokens + kBlockSize - 1) / kBlockSize;
  const long long nwork = groups * hkv;
  for (long long wk = blockIdx.x; wk < nwork; wk += gridDim.x) {
    const int h = (int)(wk % hkv);
    const long long t0 = (wk / hkv) * kBlockSize;
    const int nt = (int)min((long long)kBlockSize, num_tokens - t0);
    // every wave reads the group's slots (lane % 16) and decides the path itself
    const int j = lane & 15;
    const long long my_slot = j < nt ? (long long)slots[t0 + j] : -1;
    const long long slot0 = __shfl(my_slot, 0);
    const bool in_order = nt == kBlockSize && slot0 >= 0 && slot0 % kBlockSize == 0 &&
                          slot0 + kBlockSize <= num_slots && my_slot == slot0 + j;
    const bool aligned = __all(in_order);
    // piece p of K (and of V in order): token p / CH, chunk p % CH.  Scattered V piece p:
    // token p % 16, chunk p / 16.  Every lane runs the same trip count so that the
    // shuffles find their source lanes active.
    uint4 kx[NP], vx[NP];
    long long ksl[NP], vsl[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = i * 256 + tid;
      const int kj = min(p / CH, kBlockSize - 1), vj = aligned ? kj : p % kBlockSize;
      ksl[i] = __shfl(my_slot, kj);
      vsl[i] = __shfl(my_slot, vj);
      const int vc = aligned ? p % CH : p / kBlockSize;
      if (p < PG && kj < nt && ksl[i] >= 0 && ksl[i] < num_slots)
        kx[i] = *reinterpret_cast<const uint4*>(k + ((t0 + kj) * hkv + h) * D + (p % CH) * VEC);
      if (p < PG && vj < nt && vsl[i] >= 0 && vsl[i] < num_slots)
        vx[i] = *reinterpret_cast<const uint4*>(v + ((t0 + vj) * hkv + h) * D + vc * VEC);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = i * 256 + tid;
      const int kj = min(p / CH, kBlockSize - 1);
      if (p < PG && kj < nt && ksl[i] >= 0 && ksl[i] < num_slots)
        *reinterpret_cast<uint4*>(k_pool + (((ksl[i] / kBlockSize) * hkv + h) * kBlockSize +
                                            ksl[i] % kBlockSize) * D + (p % CH) * VEC) = kx[i];
    }
    if (aligned) {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int p = i * 256 + tid;
        if (p < PG) *reinterpret_cast<uint4*>(vs + p * VEC) = vx[i];  // [token][d]
      }
      __syncthreads();
      // V^T piece q: d row q / UPR, keys (q % UPR) * VEC ..
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int q = i * 256 + tid;
        if (q < PG) {
          const int dd = q / UPR, u = q % UPR;
          union {
            uint4 u4;
            T e[VEC];
          } run;
#pragma unroll
          for (int e = 0; e < VEC; ++e) run.e[e] = vs[(u * VEC + e) * D + dd];
          *reinterpret_cast<uint4*>(
              v_pool + (((slot0 / kBlockSize) * hkv + h) * D + dd) * kBlockSize + u * VEC) =
              run.u4;
        }
      }
      __syncthreads();  // the stage is refilled by this workgroup's next group
    } else {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int p = i * 256 + tid;
        const int vj = p % kBlockSize, c = p / kBlockSize;
        if (p < PG && vj < nt && vsl[i] >= 0 && vsl[i] < num_slots) {
          union {
            uint4 u4;
            T e[VEC];
          } x;
          x.u4 = vx[i];
          T* dst = v_pool + (((vsl[i] / kBlockSize) * hkv + h) * D + c * VEC) * kBlockSize +
                   vsl[i] % kBlockSize;
#pragma unroll
          for (int e = 0; e < VEC; ++e) dst[e * kBlockSize] = x.e[e];
        }
      }
    }
  }
}

template <typename T>
static int launch_cache_write(const void* k, const void* v, const int32_t* slots, int n, int hkv,
                              int d, void* kp, void* vp, long long num_slots, hipStream_t s) {
  long long blocks = ((long long)n + kBlockSize - 1) / kBlockSize * hkv;
  if (blocks > 65536) blocks = 65536;
  if (d == 128)
    hipLaunchKernelGGL((cache_write_kernel<T, 128>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const T*)k, (const T*)v, slots, (long long)n, hkv, (T*)kp, (T*)vp,
                       num_slots);
  else
    hipLaunchKernelGGL((cache_write_kernel<T, 64>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const T*)k, (const T*)v, slots, (long long)n, hkv, (T*)kp, (T*)vp,
                       num_slots);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

// The conventional write of a RoPE cache, kept for the in-kernel-rotation
// ablation: the key is rotated to its position before it is stored (rotate-
// half pairs (i, i + d/2), angle table from pic_rope_table), so the block is
// only valid at that one offset.  One thread per (token, head, VEC pairs):
// it reads the two halves of the pairs, writes both rotated halves, and
// copies the same elements of V unchanged.  The rotation is computed in fp32
// with the same expression the attention kernels use, then rounded to T.
template <typename T>
__global__ void __launch_bounds__(256) cache_write_rotated_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ positions, const float* __restrict__ cos_tab,
    const float* __restrict__ sin_tab, int max_pos, long long num_tokens, int hkv, int head_dim,
    T* __restrict__ k_pool, T* __restrict__ v_pool, long long num_slots) {
  constexpr int VEC = 16 / sizeof(T);
  const int half = head_dim / 2;
  const int chunks = half / VEC;  // chunks of the first half of d
  const long long n = num_tokens * hkv * chunks;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * 256) {
    const int c = (int)(idx % chunks);
    const long long th = idx / chunks;  // token * hkv + head
    const int h = (int)(th % hkv);
    const long long t = th / hkv;
    const long long slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int p = min(max(positions[t], 0), max_pos - 1);
    const long long blk = slot / kBlockSize;
    const int off = (int)(slot % kBlockSize);
    const int i0 = c * VEC;
    T* kdst = k_pool + ((blk * hkv + h) * kBlockSize + off) * head_dim;
    T* vdst = v_pool + (blk * hkv + h) * (long long)head_dim * kBlockSize + off;
    const T* ks = k + th * head_dim;
    const T* vs = v + th * head_dim;
    const float* cr = cos_tab + (long long)p * half + i0;
    const float* sr = sin_tab + (long long)p * half + i0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float x = (float)ks[i0 + e], y = (float)ks[half + i0 + e];
      const float co = cr[e], si = sr[e];
      kdst[i0 + e] = (T)(x * co - y * si);
      kdst[half + i0 + e] = (T)(y * co + x * si);
      vdst[(long long)(i0 + e) * kBlockSize] = vs[i0 + e];
      vdst[(long long)(half + i0 + e) * kBlockSize] = vs[half + i0 + e];
    }
  }
}

template <typename T>
static int launch_cache_write_rotated(const void* k, const void* v, const int32_t* slots,
                                      const int32_t* positions, const float* cos_tab,
                                      const float* sin_tab, int max_pos, int n, int hkv, int d,
                                      void* kp, void* vp, long long num_slots, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  const long long nt = (long long)n * hkv * (d / 2 / VEC);
  long long blocks = (nt + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(cache_write_rotated_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const T*)k, (const T*)v, slots, positions, cos_tab, sin_tab, max_pos,
                     (long long)n, hkv, d, (T*)kp, (T*)vp, num_slots);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

// Whole-block copies between two pools, for moving position-free blocks
// between GPU memory and pinned host memory (MiniPIC §3, contribution 5:
// unrotated blocks move between GPU and host with no position bookkeeping).
// Either pool may live in device memory or in pinned host memory that the
// device can address.  One thread per 16 bytes of a block: the (K, V) bytes of
// block src_ids[i] of the source go to block dst_ids[i] of the destination;
// K and V of one block are each hkv * B * d contiguous elements, so the copy
// is a contiguous 16-byte stream per block pair.  Pairs with an id out of
// range are skipped.
__global__ void __launch_bounds__(256) blocks_copy_kernel(
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v,
    const int32_t* __restrict__ src_ids, uint4* __restrict__ dst_k, uint4* __restrict__ dst_v,
    const int32_t* __restrict__ dst_ids, long long n_pairs, long long chunks_per_block,
    int num_src, int num_dst) {
  const long long n = n_pairs * chunks_per_block;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * 256) {
    const long long i = idx / chunks_per_block;
    const long long c = idx % chunks_per_block;
    const int sb = src_ids[i], db = dst_ids[i];
    if (sb < 0 || sb >= num_src || db < 0 || db >= num_dst) continue;
    dst_k[(long long)db * chunks_per_block + c] = src_k[(long long)sb * chunks_per_block + c];
    dst_v[(long long)db * chunks_per_block + c] = src_v[(long long)sb * chunks_per_block + c];
  }
}

}  // namespace pic

extern "C" int pic_cache_write(const void* k, const void* v, const int32_t* slot_mapping,
                               int num_tokens, int num_kv_heads, int head_dim, int dtype,
                               void* k_pool, void* v_pool, int num_blocks, int block_size,
                               void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return PIC_EINVAL;
  if (dtype != PIC_F32 && dtype != PIC_BF16) return PIC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PIC_EUNSUPPORTED;
  if (block_size != pic::kBlockSize) return PIC_EUNSUPPORTED;
  if (num_tokens == 0) return PIC_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PIC_EINVAL;
  const long long num_slots = (long long)num_blocks * block_size;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PIC_BF16)
    return pic::launch_cache_write<uint16_t>(k, v, slot_mapping, num_tokens,
                                              num_kv_heads, head_dim, k_pool, v_pool,
                                              num_slots, s);
  return pic::launch_cache_write<float>(k, v, slot_mapping, num_tokens, num_kv_heads, head_dim,
                                        k_pool, v_pool, num_slots, s);
}

extern "C" int pic_cache_write_rotated(const void* k, const void* v, const int32_t* slot_mapping,
                                       const int32_t* positions, const float* cos_tab,
                                       const float* sin_tab, int max_pos, int num_tokens,
                                       int num_kv_heads, int head_dim, int dtype, void* k_pool,
                                       void* v_pool, int num_blocks, int block_size,
                                       void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0 || max_pos <= 0) return PIC_EINVAL;
  if (dtype != PIC_F32 && dtype != PIC_BF16) return PIC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PIC_EUNSUPPORTED;
  if (block_size != pic::kBlockSize) return PIC_EUNSUPPORTED;
  if (num_tokens == 0) return PIC_OK;
  if (!k || !v || !slot_mapping || !positions || !cos_tab || !sin_tab || !k_pool || !v_pool)
    return PIC_EINVAL;
  const long long num_slots = (long long)num_blocks * block_size;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == PIC_BF16)
    return pic::launch_cache_write_rotated<__bf16>(k, v, slot_mapping, positions, cos_tab,
                                                   sin_tab, max_pos, num_tokens, num_kv_heads,
                                                   head_dim, k_pool, v_pool, num_slots, s);
  return pic::launch_cache_write_rotated<float>(k, v, slot_mapping, positions, cos_tab, sin_tab,
                                                max_pos, num_tokens, num_kv_heads, head_dim,
                                                k_pool, v_pool, num_slots, s);
}

extern "C" int pic_blocks_copy(const void* src_k_pool, const void* src_v_pool,
                               const int32_t* src_blocks, int num_src_blocks, void* dst_k_pool,
                               void* dst_v_pool, const int32_t* dst_blocks, int num_dst_blocks,
                               int num_pairs, int num_kv_heads, int head_dim, int dtype,
                               int block_size, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || num_src_blocks < 0 || num_dst_blocks < 0)
    return PIC_EINVAL;
  if (dtype != PIC_F32 && dtype != PIC_BF16) return PIC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PIC_EUNSUPPORTED;
  if (block_size != pic::kBlockSize) return PIC_EUNSUPPORTED;
  if (num_pairs == 0) return PIC_OK;
  if (!src_k_pool || !src_v_pool || !src_blocks || !dst_k_pool || !dst_v_pool || !dst_blocks)
    return PIC_EINVAL;
  const long long elem = dtype == PIC_BF16 ? 2 : 4;
  const long long chunks = (long long)num_kv_heads * block_size * head_dim * elem / 16;
  const long long n = (long long)num_pairs * chunks;
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pic::blocks_copy_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, (const uint4*)src_k_pool, (const uint4*)src_v_pool,
                     src_blocks, (uint4*)dst_k_pool, (uint4*)dst_v_pool, dst_blocks,
                     (long long)num_pairs, chunks, num_src_blocks, num_dst_blocks);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

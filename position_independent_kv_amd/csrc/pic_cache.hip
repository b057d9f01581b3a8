// pic_cache_write: store new tokens' keys and values, unrotated, into the pools.
//
// MiniPIC §2.1: the cache holds non-rotated key vectors k~_j, which is what
// lets one physical block serve requests at different offsets without being
// rewritten.  This is a pure scatter: the stored bytes are the input bytes.
//
// K goes to k_pool[block][h][offset][d] (one contiguous row per token and
// head): a flat, coalesced 16-byte copy.  V goes to v_pool[block][h][d][offset]
// (transposed inside the block so that the attention kernels read runs of
// consecutive keys as matrix-core operands): lanes take consecutive tokens,
// so tokens that share a block write neighbouring bytes of each d row.
#include <hip/hip_runtime.h>

#include "pic.h"
#include "pic_common.hpp"

namespace pic {

// One thread per (token, head, 16-byte chunk of the row).
template <typename T>
__global__ void __launch_bounds__(256) cache_write_k_kernel(const T* __restrict__ k,
                                                            const int32_t* __restrict__ slots,
                                                            long long num_tokens, int hkv,
                                                            int head_dim,
                                                            T* __restrict__ k_pool,
                                                            long long num_slots) {
  constexpr int VEC = 16 / sizeof(T);
  const int chunks = head_dim / VEC;
  const long long n = num_tokens * hkv * chunks;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * 256) {
    const int c = (int)(idx % chunks);
    const long long th = idx / chunks;  // token * hkv + head
    const int h = (int)(th % hkv);
    const long long t = th / hkv;
    const long long slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const long long blk = slot / kBlockSize;
    const int off = (int)(slot % kBlockSize);
    const uint4 x = *reinterpret_cast<const uint4*>(k + th * head_dim + c * VEC);
    *reinterpret_cast<uint4*>(k_pool + ((blk * hkv + h) * kBlockSize + off) * head_dim +
                              c * VEC) = x;
  }
}

// One wave per (64 consecutive tokens, head); lane = token.
template <typename T>
__global__ void __launch_bounds__(256) cache_write_v_kernel(const T* __restrict__ v,
                                                            const int32_t* __restrict__ slots,
                                                            long long num_tokens, int hkv,
                                                            int head_dim,
                                                            T* __restrict__ v_pool,
                                                            long long num_slots) {
  constexpr int VEC = 16 / sizeof(T);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const long long waves_total = (long long)gridDim.x * 4;
  const long long tiles = ((num_tokens + 63) / 64) * hkv;
  for (long long w = (long long)blockIdx.x * 4 + wave; w < tiles; w += waves_total) {
    const int h = (int)(w % hkv);
    const long long t = (w / hkv) * 64 + lane;
    if (t >= num_tokens) continue;
    const long long slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const long long blk = slot / kBlockSize;
    const int off = (int)(slot % kBlockSize);
    const T* src = v + (t * hkv + h) * head_dim;
    T* dst = v_pool + (blk * hkv + h) * (long long)head_dim * kBlockSize + off;
    for (int e = 0; e < head_dim; e += VEC) {
      const uint4 x = *reinterpret_cast<const uint4*>(src + e);
      const T* xs = reinterpret_cast<const T*>(&x);
#pragma unroll
      for (int j = 0; j < VEC; ++j) dst[(long long)(e + j) * kBlockSize] = xs[j];
    }
  }
}

template <typename T>
static int launch_cache_write(const void* k, const void* v, const int32_t* slots, int n, int hkv,
                              int d, void* kp, void* vp, long long num_slots, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  const long long nk = (long long)n * hkv * (d / VEC);
  long long bk = (nk + 255) / 256;
  if (bk > 65536) bk = 65536;
  hipLaunchKernelGGL(cache_write_k_kernel<T>, dim3((unsigned)bk), dim3(256), 0, s,
                     (const T*)k, slots, (long long)n, hkv, d, (T*)kp, num_slots);
  const long long tiles = ((long long)(n + 63) / 64) * hkv;
  long long bv = (tiles + 3) / 4;
  if (bv > 65536) bv = 65536;
  hipLaunchKernelGGL(cache_write_v_kernel<T>, dim3((unsigned)bv), dim3(256), 0, s,
                     (const T*)v, slots, (long long)n, hkv, d, (T*)vp, num_slots);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
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

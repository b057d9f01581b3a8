// pic_stream_read: plain streaming reads of device memory, the ceilings the
// memory-bound decode path is measured against on the same machine.  The
// buffer is read as 4 KiB segments (256 lanes x 16 bytes), each workgroup
// taking U segments per iteration (U loads in flight per lane), grid-stride.
// Without an order the segments are read front to back; with one, the buffer
// is a list of pieces of piece_bytes (a multiple of 4 KiB) read whole in the
// listed order, which is how a paged cache's randomly placed blocks are read.
// The data is folded into one word per lane, stored only when it equals a
// fixed constant, so no load can be dropped and (almost) nothing is written.
#include <hip/hip_runtime.h>

#include "pic.h"

namespace pic {

constexpr int kStreamUnroll = 8;
constexpr long long kSegBytes = 4096;

template <int U>
__global__ void __launch_bounds__(256) stream_read_kernel(const uint4* __restrict__ src,
                                                          long long nseg,
                                                          const int32_t* __restrict__ order,
                                                          long long seg_per_piece,
                                                          unsigned* __restrict__ sink) {
  const unsigned long long last_piece = (unsigned long long)(nseg / seg_per_piece) - 1;
  unsigned acc = 0;
  for (long long s0 = (long long)blockIdx.x * U; s0 < nseg; s0 += (long long)gridDim.x * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long s = s0 + u;
      long long seg = s;
      if (order && s < nseg) {  // an entry outside the buffer reads its last piece
        const unsigned long long piece =
            min((unsigned long long)(unsigned)order[s / seg_per_piece], last_piece);
        seg = (long long)piece * seg_per_piece + s % seg_per_piece;
      }
      v[u] = s < nseg ? src[seg * (kSegBytes / 16) + threadIdx.x] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[(long long)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace pic

extern "C" int pic_stream_read(const void* src, size_t bytes, const int32_t* order,
                               int piece_bytes, int workgroups, void* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % pic::kSegBytes || workgroups <= 0 ||
      workgroups > (1 << 20))
    return PIC_EINVAL;
  long long seg_per_piece = 1;
  if (order) {
    if (piece_bytes <= 0 || piece_bytes % pic::kSegBytes || bytes % (size_t)piece_bytes)
      return PIC_EINVAL;
    seg_per_piece = piece_bytes / pic::kSegBytes;
  }
  hipLaunchKernelGGL(pic::stream_read_kernel<pic::kStreamUnroll>, dim3((unsigned)workgroups),
                     dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                     (long long)(bytes / pic::kSegBytes), order, seg_per_piece, (unsigned*)sink);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

// pic_rope_table: the cosine/sine lookup table the attention kernels read.
//
// MiniPIC §2.1 (Implementation bullet): the position-free kernel looks up a
// cosine/sine table and does fused multiply-adds for every key element.  The
// page does not give the frequencies; this library uses the standard rotary
// ones, theta_i = base^(-2i/d).  Angles p * theta_i reach 1.3e5 rad at the
// longest contexts, so they and the trig functions are evaluated in float64;
// the table is stored in float32.
#include <hip/hip_runtime.h>

#include "pic.h"
#include "pic_common.hpp"

namespace pic {

__global__ void __launch_bounds__(256) rope_table_kernel(float* __restrict__ cos_tab,
                                                         float* __restrict__ sin_tab,
                                                         int max_pos, int head_dim,
                                                         double base) {
  const int half = head_dim / 2;
  const long long n = (long long)max_pos * half;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * 256) {
    const int p = (int)(idx / half);
    const int i = (int)(idx % half);
    const double theta = pow(base, -2.0 * (double)i / (double)head_dim);
    const double ang = (double)p * theta;
    double s, c;
    sincos(ang, &s, &c);
    cos_tab[idx] = (float)c;
    sin_tab[idx] = (float)s;
  }
}

}  // namespace pic

extern "C" int pic_rope_table(float* cos_tab, float* sin_tab, int max_pos, int head_dim,
                              double base, void* stream) {
  if (!cos_tab || !sin_tab || max_pos <= 0 || !(base > 0.0)) return PIC_EINVAL;
  if (head_dim <= 0 || head_dim % 2) return PIC_EUNSUPPORTED;
  const long long n = (long long)max_pos * (head_dim / 2);
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pic::rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, cos_tab, sin_tab, max_pos, head_dim, base);
  return hipGetLastError() == hipSuccess ? PIC_OK : PIC_EHIP;
}

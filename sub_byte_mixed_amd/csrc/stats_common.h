// Statistics finalisation shared by the quantizer launches (finalize_kernel)
// and the GEMM launches that carry it as extra workgroups: one workgroup of
// 256 threads sums one tensor's per-workgroup partials in a fixed order.
//
// "SNIP", Abstract: activation and gradient statistics feed the precision
// decision; "FP4 All the Way" summary, Outline: the sqrt(3) noise threshold
// is judged from the tensor norm and the quantization-error norm.
#pragma once

#include "device.h"
#include "kernels.h"

namespace snip {

__device__ inline void finalize_one(const FJob& J) {
  double e2 = 0.0, x2 = 0.0;
  uint32_t nf = 0u, am = 0u;
  for (int i = threadIdx.x; i < J.nwg; i += 256) {
    const StatPart p = J.part[i];
    e2 += p.e2;
    x2 += p.x2;
    nf += p.nf;
    am = p.amax_bits > am ? p.amax_bits : am;
  }
  __shared__ uint32_t fured[8];
  __shared__ double fdred[8];
  e2 = wave_sum(e2);
  x2 = wave_sum(x2);
  nf = wave_sum_u(nf);
  am = wave_max_u(am);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    fdred[2 * wave] = e2;
    fdred[2 * wave + 1] = x2;
    fured[2 * wave] = nf;
    fured[2 * wave + 1] = am;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    snip_stats s{0.0, 0.0, 0.0f, 0u};
    uint32_t m = 0u;
    for (int w = 0; w < 4; ++w) {
      s.sum_err2 += fdred[2 * w];
      s.sum_x2 += fdred[2 * w + 1];
      s.n_nonfinite += fured[2 * w];
      m = fured[2 * w + 1] > m ? fured[2 * w + 1] : m;
    }
    s.amax = __uint_as_float(m);
    *J.out = s;
  }
}

}  // namespace snip

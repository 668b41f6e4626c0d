// The matrix cores alone: a loop of v_mfma_i32_16x16x64_i8 with no memory
// traffic, to measure the int8 MFMA rate this chip reaches in practice (the
// ceiling the grouped expert GEMMs are compared with beside the published
// dense peak).  Each wave runs 8 independent accumulator chains, so that
// the issue of one MFMA never waits on the result of the previous one.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef int v4i_pk __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) k_mfma_peak(int iters, int32_t *out) {
  const int lane = threadIdx.x & 63;
  // operand byte j of lane l: (7 l + 3 j) mod 4 and (5 l + j) mod 3, so each
  // MFMA adds at most 64 * 3 * 2 = 384 to an element: no int32 overflow for
  // iters < 2^21
  uint32_t aw[4], bw[4];
#pragma unroll
  for (int w = 0; w < 4; w++) {
    aw[w] = bw[w] = 0u;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int j = 4 * w + q;
      aw[w] |= (uint32_t)((7 * lane + 3 * j) & 3) << (8 * q);
      bw[w] |= (uint32_t)((5 * lane + j) % 3) << (8 * q);
    }
  }
  const v4i_pk a = {(int)aw[0], (int)aw[1], (int)aw[2], (int)aw[3]};
  const v4i_pk b = {(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3]};
  v4i_pk acc[8];
#pragma unroll
  for (int c = 0; c < 8; c++) acc[c] = v4i_pk{c, 0, 0, 0};
  for (int i = 0; i < iters; i++) {
#pragma unroll
    for (int c = 0; c < 8; c++) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int c = 0; c < 8; c++) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

void launch_mfma_peak(int n_wg, int iters, int32_t *out, hipStream_t st) {
  hipLaunchKernelGGL(k_mfma_peak, dim3(n_wg), dim3(256), 0, st, iters, out);
}

}  // namespace moe

// Measurement loops.  The matrix cores alone: a loop of v_mfma_i32_16x16x64_i8 with no memory
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

// HBM alone: a plain streaming read of n16 16-byte pieces with the expert
// kernels' own non-temporal loads, four in flight per thread (grid-stride),
// to measure the read rate this chip reaches for a given byte count (the
// ceiling the HBM-bound expert kernels are compared with beside the
// published peak).  Each wave XORs its words into one checksum word, so no
// load is elided.
__global__ void __launch_bounds__(256) k_read_peak(const uint8_t *buf, int64_t n16, uint32_t *out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) v[u] = gload_stream(buf, (size_t)(i + u * stride) * 16);
#pragma unroll
    for (int u = 0; u < 4; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = gload_stream(buf, (size_t)i * 16);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) out[(size_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

void launch_read_peak(const void *buf, int64_t bytes, int n_wg, uint32_t *out, hipStream_t st,
                      Ev ev) {
  launch_k(k_read_peak, dim3(n_wg), dim3(256), 0, st, ev, static_cast<const uint8_t *>(buf),
           bytes / 16, out);
}

}  // namespace moe

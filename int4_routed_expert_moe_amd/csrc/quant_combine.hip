// Q8_0 activation quantiser, weighted combine and RMSNorm.
//
// Q8_0 follows the int8-activation item of "Show HN: 遅いコンピュータで GLM 5.2
// を実行する" (section 実装済みの主な機能): blocks of 32 values, one fp32 scale
// d = amax/127 per block, codes roundf(x * (1/d)) in [-127, 127].
// The combine is the router item of the same list: routed outputs weighted by
// the normalised, routed_scaling_factor-scaled gates, plus the shared expert.
#include "common.h"
#include "kernels.h"

namespace moe {

// 8 lanes per 32-element block, 4 consecutive floats per lane.  Memory
// traffic is one coalesced float4 read and one 4-byte write per lane.
__global__ void __launch_bounds__(256) k_quant_act(const float *__restrict__ x,
                                                   int8_t *__restrict__ q,
                                                   float *__restrict__ d, int64_t n_quads) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = i < n_quads;
  float4 v = live ? reinterpret_cast<const float4 *>(x)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  a = fmaxf(a, __shfl_xor(a, 1, 8));
  a = fmaxf(a, __shfl_xor(a, 2, 8));
  a = fmaxf(a, __shfl_xor(a, 4, 8));
  const float dd = a / 127.0f;
  const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
  if (!live) return;
  auto cv = [&](float f) -> uint32_t {
    float r = roundf(f * id);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(uint8_t)(int8_t)(int)r;
  };
  uint32_t packed = cv(v.x) | (cv(v.y) << 8) | (cv(v.z) << 16) | (cv(v.w) << 24);
  reinterpret_cast<uint32_t *>(q)[i] = packed;
  if ((i & 7) == 0) d[i >> 3] = dd;
}

void launch_quant_act(const float *x, int8_t *q, float *d, int64_t n_elems, hipStream_t st,
                      const moe_events *ev) {
  const int64_t quads = n_elems / 4;
  const int64_t blocks = (quads + 255) / 256;
  launch_k(k_quant_act, dim3((unsigned)blocks), dim3(256), 0, st, stage_ev(ev, MOE_STAGE_QUANT), x,
           q, d, quads);
}

// The per-row activation format (one scale per row, the Q8_0 rule over the
// whole row): one workgroup per row of n floats (n % 4 == 0).  The row's
// amax (a maximum, so exact in any order), then d = amax/127,
// id = d != 0 ? 1/d : 0, q = clamp(roundf(x * id), -127, 127).  Rows
// r < n_skip whose skip[r] < 0 (slots dropped by top-p) are left alone.
__global__ void __launch_bounds__(256) k_quant_rows(const float *__restrict__ x,
                                                    int8_t *__restrict__ q,
                                                    float *__restrict__ d, int n,
                                                    const int32_t *__restrict__ skip,
                                                    int n_skip) {
  __shared__ float wm[4];
  const size_t row = blockIdx.x;
  if (skip && (int)row < n_skip && skip[row] < 0) return;
  const float4 *x4 = reinterpret_cast<const float4 *>(x + row * n);
  uint32_t *q4 = reinterpret_cast<uint32_t *>(q + row * n);
  const int n4 = n / 4;
  float m = 0.0f;
  for (int i = threadIdx.x; i < n4; i += 256) {
    const float4 v = x4[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  const float dd = amax / 127.0f;
  const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
  auto cv = [&](float f) -> uint32_t {
    float r = roundf(f * id);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(uint8_t)(int8_t)(int)r;
  };
  for (int i = threadIdx.x; i < n4; i += 256) {
    const float4 v = x4[i];
    q4[i] = cv(v.x) | (cv(v.y) << 8) | (cv(v.z) << 16) | (cv(v.w) << 24);
  }
  if (threadIdx.x == 0) d[row] = dd;
}

void launch_quant_rows(const float *x, int8_t *q, float *d, int64_t rows, int n,
                       const int32_t *skip, int n_skip, hipStream_t st, const moe_events *ev) {
  if (rows <= 0) return;
  launch_k(k_quant_rows, dim3((unsigned)rows), dim3(256), 0, st, stage_ev(ev, MOE_STAGE_QUANT), x, q,
           d, n, skip, n_skip);
}

// y = residual + shared + sum_k w_k * expert_k (fp32, rank order); the
// optional unit-gain RMSNorm of y is a second kernel (k_rmsnorm).
// Workgroup (t, c): values 1024 c .. 1024 c + 1023 of token t's output (one
// float4 per thread), so that a few tokens still spread over many CUs.
__global__ void __launch_bounds__(256) k_combine(int H, int K, const float *__restrict__ eo,
                                                 const float *__restrict__ w,
                                                 const float *__restrict__ shared,
                                                 const float *__restrict__ residual,
                                                 float *__restrict__ y) {
  const int t = blockIdx.x, j = blockIdx.y * 256 + threadIdx.x;
  const int H4 = H / 4;
  __shared__ float wk[16];
  if (threadIdx.x < K) wk[threadIdx.x] = w[(size_t)t * K + threadIdx.x];
  __syncthreads();
  if (j >= H4) return;
  const float4 *eo4 = reinterpret_cast<const float4 *>(eo) + (size_t)t * K * H4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (residual) acc = reinterpret_cast<const float4 *>(residual)[(size_t)t * H4 + j];
  if (shared) {
    float4 s = reinterpret_cast<const float4 *>(shared)[(size_t)t * H4 + j];
    acc.x += s.x; acc.y += s.y; acc.z += s.z; acc.w += s.w;
  }
  for (int k0 = 0; k0 < K; k0 += 8) {
    // 8 ranks' rows requested at once (one memory round trip, not 8); a rank
    // dropped by top-p (weight 0, its row never written) is read and skipped
    float4 e[8];
#pragma unroll
    for (int u = 0; u < 8; u++) e[u] = eo4[(size_t)min(k0 + u, K - 1) * H4 + j];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const float c = k0 + u < K ? wk[k0 + u] : 0.0f;
      if (c != 0.0f) {
        acc.x = fmaf(c, e[u].x, acc.x);
        acc.y = fmaf(c, e[u].y, acc.y);
        acc.z = fmaf(c, e[u].z, acc.z);
        acc.w = fmaf(c, e[u].w, acc.w);
      }
    }
  }
  reinterpret_cast<float4 *>(y)[(size_t)t * H4 + j] = acc;
}

// RMSNorm, workgroup (t, c): the sum of squares of token t's whole row (read
// by every workgroup of the row, four loads in flight per thread), then
// values 1024 c .. 1024 c + 1023 scaled.
__global__ void __launch_bounds__(256) k_rmsnorm(int H, const float *__restrict__ x,
                                                 float *__restrict__ y, float eps) {
  const int t = blockIdx.x, jc = blockIdx.y * 256 + threadIdx.x;
  const int H4 = H / 4;
  __shared__ float red[4];
  const float4 *x4 = reinterpret_cast<const float4 *>(x) + (size_t)t * H4;
  float ss = 0.0f;
  for (int j0 = 0; j0 < H4; j0 += 1024) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int j = j0 + u * 256 + threadIdx.x;
      v[u] = j < H4 ? x4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) ss += v[u].x * v[u].x + v[u].y * v[u].y + v[u].z * v[u].z + v[u].w * v[u].w;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  if (jc < H4) {
    float4 v = x4[jc];
    v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
    reinterpret_cast<float4 *>(y)[(size_t)t * H4 + jc] = v;
  }
}

void launch_combine(int T, int H, int K, const float *eo, const float *w, const float *shared,
                    const float *residual, float *y, float *yn, float eps, hipStream_t st,
                    const moe_events *ev) {
  const Ev e = stage_ev(ev, MOE_STAGE_COMBINE);
  const dim3 g(T, (H / 4 + 255) / 256);
  launch_k(k_combine, g, dim3(256), 0, st, Ev{e.start, yn ? nullptr : e.stop}, H, K, eo, w,
           shared, residual, y);
  if (yn) launch_k(k_rmsnorm, g, dim3(256), 0, st, Ev{nullptr, e.stop}, H, (const float *)y, yn, eps);
}

void launch_rmsnorm(int T, int H, const float *x, float *y, float eps, hipStream_t st) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(T, (H / 4 + 255) / 256), dim3(256), 0, st, H, x, y, eps);
}

}  // namespace moe

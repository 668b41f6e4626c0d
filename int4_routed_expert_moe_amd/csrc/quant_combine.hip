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

// One block per token row; 256 threads stride over H in float4.
// y = residual + shared + sum_k w_k * expert_k (fp32, rank order); optional
// unit-gain RMSNorm of y.
__global__ void __launch_bounds__(256) k_combine(int H, int K, const float *__restrict__ eo,
                                                 const float *__restrict__ w,
                                                 const float *__restrict__ shared,
                                                 const float *__restrict__ residual,
                                                 float *__restrict__ y, float *__restrict__ yn,
                                                 float eps) {
  const int t = blockIdx.x;
  const int H4 = H / 4;
  __shared__ float wk[16];
  __shared__ float red[4];
  if (threadIdx.x < K) wk[threadIdx.x] = w[(size_t)t * K + threadIdx.x];
  __syncthreads();
  float ss = 0.0f;
  const float4 *eo4 = reinterpret_cast<const float4 *>(eo) + (size_t)t * K * H4;
  for (int j = threadIdx.x; j < H4; j += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (residual) acc = reinterpret_cast<const float4 *>(residual)[(size_t)t * H4 + j];
    if (shared) {
      float4 s = reinterpret_cast<const float4 *>(shared)[(size_t)t * H4 + j];
      acc.x += s.x; acc.y += s.y; acc.z += s.z; acc.w += s.w;
    }
    for (int k = 0; k < K; k++) {
      const float c = wk[k];
      if (c == 0.0f) continue;  // a rank dropped by top-p: its row is not read
      float4 e = eo4[(size_t)k * H4 + j];
      acc.x = fmaf(c, e.x, acc.x);
      acc.y = fmaf(c, e.y, acc.y);
      acc.z = fmaf(c, e.z, acc.z);
      acc.w = fmaf(c, e.w, acc.w);
    }
    reinterpret_cast<float4 *>(y)[(size_t)t * H4 + j] = acc;
    ss += acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w;
  }
  if (!yn) return;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  for (int j = threadIdx.x; j < H4; j += 256) {
    float4 v = reinterpret_cast<const float4 *>(y)[(size_t)t * H4 + j];
    v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
    reinterpret_cast<float4 *>(yn)[(size_t)t * H4 + j] = v;
  }
}

void launch_combine(int T, int H, int K, const float *eo, const float *w, const float *shared,
                    const float *residual, float *y, float *yn, float eps, hipStream_t st,
                    const moe_events *ev) {
  launch_k(k_combine, dim3(T), dim3(256), 0, st, stage_ev(ev, MOE_STAGE_COMBINE), H, K, eo, w,
           shared, residual, y, yn, eps);
}

__global__ void __launch_bounds__(256) k_rmsnorm(int H, const float *__restrict__ x,
                                                 float *__restrict__ y, float eps) {
  const int t = blockIdx.x;
  const int H4 = H / 4;
  __shared__ float red[4];
  const float4 *x4 = reinterpret_cast<const float4 *>(x) + (size_t)t * H4;
  float ss = 0.0f;
  for (int j = threadIdx.x; j < H4; j += 256) {
    float4 v = x4[j];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  for (int j = threadIdx.x; j < H4; j += 256) {
    float4 v = x4[j];
    v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
    reinterpret_cast<float4 *>(y)[(size_t)t * H4 + j] = v;
  }
}

void launch_rmsnorm(int T, int H, const float *x, float *y, float eps, hipStream_t st) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, st, H, x, y, eps);
}

}  // namespace moe

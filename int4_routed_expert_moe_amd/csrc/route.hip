// Router: sigmoid scores and noaux_tc group-limited top-k.
//
// Follows the router item of "Show HN: 遅いコンピュータで GLM 5.2 を実行する"
// (ja.news.hada.io, section 実装済みの主な機能): a DeepSeek-V3-style sigmoid
// router with noaux_tc selection and routed_scaling_factor.  The correction
// bias takes part in selection only; the routing weights are the unbiased
// sigmoid scores of the chosen experts, normalised and scaled.
//
// The fp32 arithmetic of the scores is fixed so that the chosen indices are
// a function of the inputs alone (the same steps on a CPU give the same
// bits): the dot product runs over consecutive 64-element chunks, each an fma
// chain in increasing index starting from 0, and the chunk partials are
// added left to right; e^y is a Cody–Waite reduction by ln 2 (split in a
// 16-bit high part and a low part) followed by the degree-7 Taylor polynomial
// of e^r in Horner form with fma, scaled by 2^n.  This file is compiled with
// -ffp-contract=off and correctly rounded fp32 division.
#include "common.h"
#include "kernels.h"

namespace moe {

// One wave per (expert, chunk of TT tokens).  Lane l owns the 64-element
// chunks l, l+64, ...; each chunk is an fma chain over its 64 elements; the
// chunk partials go to LDS and one lane per token adds them left to right.
template <int TT>
__global__ void __launch_bounds__(64) k_router_scores(int T, int H, int E,
                                                      const float *__restrict__ x,
                                                      const float *__restrict__ wr,
                                                      const float *__restrict__ bias,
                                                      float *__restrict__ s,
                                                      float *__restrict__ sb) {
  extern __shared__ float part[];  // [TT][nchunk]
  const int e = blockIdx.x, t0 = blockIdx.y * TT, lane = threadIdx.x;
  const int nchunk = H / 64;
  const float *wrow = wr + (size_t)e * H;
  for (int c = lane; c < nchunk; c += 64) {
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) acc[t] = 0.0f;
    const float4 *w4 = reinterpret_cast<const float4 *>(wrow + c * 64);
#pragma unroll 4
    for (int k4 = 0; k4 < 16; k4++) {
      const float4 wv = w4[k4];
#pragma unroll
      for (int t = 0; t < TT; t++) {
        if (t0 + t < T) {
          const float4 xv =
              reinterpret_cast<const float4 *>(x + (size_t)(t0 + t) * H + c * 64)[k4];
          acc[t] = __builtin_fmaf(xv.x, wv.x, acc[t]);
          acc[t] = __builtin_fmaf(xv.y, wv.y, acc[t]);
          acc[t] = __builtin_fmaf(xv.z, wv.z, acc[t]);
          acc[t] = __builtin_fmaf(xv.w, wv.w, acc[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TT; t++) part[t * nchunk + c] = acc[t];
  }
  __syncthreads();
  if (lane < TT && t0 + lane < T) {
    const float *p = part + lane * nchunk;
    float tot = p[0];
    for (int c = 1; c < nchunk; c++) tot = tot + p[c];
    const float sv = sigmoid_fixed(tot);
    const size_t o = (size_t)(t0 + lane) * E + e;
    s[o] = sv;
    sb[o] = sv + bias[e];
  }
}

// Router scores for larger batches as a register-tiled fp32 GEMM with the
// same fixed order: every (token, expert) output is an fma chain over each
// 64-element chunk of k in increasing order, from 0, and the chunk partials
// are added left to right.  Workgroup tile: (16 TM) tokens x (16 TN)
// experts; thread (tx, ty) owns tokens tx + 16 a and experts ty + 16 b
// (interleaved so that a wave's LDS reads fall in distinct banks).  One
// chunk of x and W (64 k each) is staged in LDS per step, rows padded to
// 68 floats, the next chunk in registers meanwhile; each thread walks k
// four at a time with 16-byte LDS reads.
namespace rg {
constexpr int KC = 64, STR = KC + 4;
}
template <int TM, int TN>
__global__ void __launch_bounds__(256) k_router_gemm(int T, int H, int E,
                                                     const float *__restrict__ x,
                                                     const float *__restrict__ wr,
                                                     const float *__restrict__ bias,
                                                     float *__restrict__ s,
                                                     float *__restrict__ sb) {
  constexpr int MT = 16 * TM, NTL = 16 * TN;
  __shared__ __align__(16) float xs[MT * rg::STR];
  __shared__ __align__(16) float ws[NTL * rg::STR];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.x * MT, e0 = blockIdx.y * NTL;
  float tot[TM][TN], acc[TM][TN];
  const int nch = H / rg::KC;
  constexpr int NX = MT * 16 / 256, NW = NTL * 16 / 256;  // float4 per thread per chunk
  float4 px[NX], pw[NW];  // the next chunk, in flight during this one's FMAs
  auto fetch = [&](int c) {
#pragma unroll
    for (int u = 0; u < NX; u++) {
      const int i = tid + 256 * u, r = i >> 4, q = i & 15, t = t0 + r;
      px[u] = t < T ? reinterpret_cast<const float4 *>(x + (size_t)t * H + c * rg::KC)[q]
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < NW; u++) {
      const int i = tid + 256 * u, r = i >> 4, q = i & 15, e = e0 + r;
      pw[u] = e < E ? reinterpret_cast<const float4 *>(wr + (size_t)e * H + c * rg::KC)[q]
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  fetch(0);
  for (int c = 0; c < nch; c++) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NX; u++) {
      const int i = tid + 256 * u;
      *reinterpret_cast<float4 *>(xs + (i >> 4) * rg::STR + (i & 15) * 4) = px[u];
    }
#pragma unroll
    for (int u = 0; u < NW; u++) {
      const int i = tid + 256 * u;
      *reinterpret_cast<float4 *>(ws + (i >> 4) * rg::STR + (i & 15) * 4) = pw[u];
    }
    __syncthreads();
    if (c + 1 < nch) fetch(c + 1);
#pragma unroll
    for (int a = 0; a < TM; a++)
#pragma unroll
      for (int b = 0; b < TN; b++) acc[a][b] = 0.0f;
#pragma unroll
    for (int k = 0; k < rg::KC; k += 4) {
      float4 xv[TM], wv[TN];
#pragma unroll
      for (int a = 0; a < TM; a++)
        xv[a] = *reinterpret_cast<const float4 *>(xs + (tx + 16 * a) * rg::STR + k);
#pragma unroll
      for (int b = 0; b < TN; b++)
        wv[b] = *reinterpret_cast<const float4 *>(ws + (ty + 16 * b) * rg::STR + k);
#pragma unroll
      for (int a = 0; a < TM; a++)
#pragma unroll
        for (int b = 0; b < TN; b++) {
          float v = acc[a][b];
          v = __builtin_fmaf(xv[a].x, wv[b].x, v);
          v = __builtin_fmaf(xv[a].y, wv[b].y, v);
          v = __builtin_fmaf(xv[a].z, wv[b].z, v);
          v = __builtin_fmaf(xv[a].w, wv[b].w, v);
          acc[a][b] = v;
        }
    }
#pragma unroll
    for (int a = 0; a < TM; a++)
#pragma unroll
      for (int b = 0; b < TN; b++) tot[a][b] = c == 0 ? acc[a][b] : tot[a][b] + acc[a][b];
  }
#pragma unroll
  for (int a = 0; a < TM; a++) {
    const int t = t0 + tx + 16 * a;
#pragma unroll
    for (int b = 0; b < TN; b++) {
      const int e = e0 + ty + 16 * b;
      if (t < T && e < E) {
        const float sv = sigmoid_fixed(tot[a][b]);
        s[(size_t)t * E + e] = sv;
        sb[(size_t)t * E + e] = sv + bias[e];
      }
    }
  }
}

// tile (16 TM tokens x 16 TN experts): 2 x 2 gives 512 workgroups at 2048
// tokens (two per CU); 2 x 4 (256 workgroups) took 197-201 us against 168,
// and 1 x 4, 1 x 2 and 4 x 2 took 194-204 us
#ifndef ROUTER_TM
#define ROUTER_TM 2
#endif
#ifndef ROUTER_TN
#define ROUTER_TN 2
#endif

void launch_router_scores(const moe_cfg &c, int T, const float *x, const float *wr,
                          const float *bias, float *s, float *sb, hipStream_t st,
                          const moe_events *ev) {
  const int H = c.hidden, E = c.n_experts;
  const Ev e0 = stage_ev(ev, MOE_STAGE_ROUTER_SCORES);
  const size_t lds = sizeof(float) * (size_t)(H / 64);
  if (T <= 1) {
    launch_k(k_router_scores<1>, dim3(E, T), dim3(64), lds, st, e0, T, H, E, x, wr, bias, s, sb);
  } else if (T <= 4) {
    launch_k(k_router_scores<4>, dim3(E, 1), dim3(64), 4 * lds, st, e0, T, H, E, x, wr, bias, s,
             sb);
  } else if (T <= 64) {
    launch_k(k_router_scores<8>, dim3(E, (T + 7) / 8), dim3(64), 8 * lds, st, e0, T, H, E, x, wr,
             bias, s, sb);
  } else {
    launch_k(k_router_gemm<ROUTER_TM, ROUTER_TN>,
             dim3((T + 16 * ROUTER_TM - 1) / (16 * ROUTER_TM),
                  (E + 16 * ROUTER_TN - 1) / (16 * ROUTER_TN)),
             dim3(256), 0, st, e0, T, H, E, x, wr, bias, s, sb);
  }
}

// The selection (group-limited top-k, weights, top-p) is the small-batch
// path's per-token selection, one workgroup per token (decode.hip,
// launch_router_select).
}  // namespace moe

// The routed-MoE layer step for small batches (decode and multi-token
// verify, 1..16 tokens) in four kernels (five with the RMSNorm of stacked layers).
//
// Same method and arithmetic as the separate calls ("Show HN: 遅いコンピュータ
// で GLM 5.2 を実行する", section 実装済みの主な機能: sigmoid router with
// noaux_tc and routed_scaling_factor, shared expert, Q8_0 int8 activations,
// packed int4/int2 weights with per-row scales, batch-union MoE), for every
// weight format: int4, int2 and int8 codes with row scales, MXFP4, and FP8
// E4M3 with 128x128 block scales (up to 4 tokens; "Comment exécuter…",
// section "Modèles supportés").
//
//  K1  k_route_small   (E workgroups) Q8_0 of a slice of x; the fixed-order
//                      fp32 logit and sigmoid score of one expert for every
//                      token (from 8 tokens: two experts, half the tokens).
//  K1b k_select_small  (T + I/4 workgroups) group-limited top-k of one token
//                      per workgroup; the rest run the shared expert's gate/up
//                      (it needs no routing), 4 rows each (one per wave), h in
//                      fp32.
//  K2  k_gate_up_small (I/32 x routed slots) each workgroup finds its expert
//                      slot of the batch union from the T*K selections, then
//                      32 rows of h = silu(gate x) * (up x) for that expert and
//                      its tokens, written directly as Q8_0 blocks (each row
//                      streamed once: a slot with more tokens than one chunk
//                      takes them from LDS); the first slot's workgroups also
//                      quantise the shared expert's h.
//  K3  k_down_small    (H/8 workgroups) 8 output rows for every expert slot
//                      and token, combined in LDS in rank order into y
//                      (+ residual), with per-tile sums of squares when the
//                      RMSNorm is wanted; from 4 tokens on (int4 and int2;
//                      MXFP4 from 8, int8 from 12) the down rows run as MFMA
//                      tiles from the slot table instead, followed by a
//                      combine kernel.
//  K4  k_norm_small    (with y_norm) the unit-gain RMSNorm of whole rows.
// Every kernel spreads its weight bytes over all CUs: one CU streams only a
// few tens of GB/s, so a phase confined to a few CUs is slow however small.
// Kernel boundaries carry every dependency; no workgroup waits for another.
#pragma once
#include "common.h"
#include "kernels.h"

#include <stddef.h>
#include <string.h>

#include <algorithm>

namespace moe {
// Every source file including this header instantiates its own copies (the
// production kernels in decode.hip, the dumping ones in decode_dbg.hip).
namespace {

// Down-kernel slot batches: a double-buffered batch (the next is requested
// while one is reduced) holds MOE_K3_SLOTS expert slots (int2 at one token:
// MOE_K3_SLOTS_INT2, measured apart for its half-length rows); formats whose registers do
// not allow two batches (bit f of MOE_K3_PIPE clear: 1 int4, 2 int2, 4 int8,
// 8 MXFP4) take MOE_K3_SLOTS_NOPIPE slots at a time.
#ifndef MOE_K3_SLOTS
#define MOE_K3_SLOTS 1
#endif
#ifndef MOE_K3_SLOTS_INT2
#define MOE_K3_SLOTS_INT2 1
#endif
#ifndef MOE_K3_SLOTS_NOPIPE
#define MOE_K3_SLOTS_NOPIPE 2
#endif
#ifndef MOE_K3_PIPE
#define MOE_K3_PIPE 0xB
#endif
// smallest batch whose router workgroups take two experts each
#ifndef MOE_ROUTE_EB2_T
#define MOE_ROUTE_EB2_T 8
#endif
// tokens per chunk of the down kernel for batches of more than one token
#ifndef MOE_K3_TT
#define MOE_K3_TT 2
#endif
// gate/up rows (each a gate and an up row) a K2 wave loads together: 1, 2, 4, 8
#ifndef MOE_K2_ROWS
#define MOE_K2_ROWS 1
#endif
// tokens per chunk of the int4 gate/up kernel for batches of more than one token
// slots with more tokens than one chunk: activations staged in LDS, rows
// streamed once
#ifndef MOE_GU_LDS
#define MOE_GU_LDS 1
#endif
#ifndef MOE_TT_INT4
#define MOE_TT_INT4 2
#endif
// shared expert rows per wave at one token (RPW1) and for batches of
// several tokens (RPW)
#ifndef MOE_SHARED_RPW1
#define MOE_SHARED_RPW1 1
#endif
#ifndef MOE_SHARED_RPW
#define MOE_SHARED_RPW 1
#endif
constexpr int shared_rpw(int TT) { return TT == 1 ? MOE_SHARED_RPW1 : MOE_SHARED_RPW; }
// tokens per chunk of the shared expert's gate/up for batches of several tokens
#ifndef MOE_SHARED_TT
#define MOE_SHARED_TT 2
#endif
// smallest batch whose down projection runs on the matrix cores (17: never):
// int4 and int2, MXFP4, and int8 (the vector down kernels of the last two
// hold out longer)
#ifndef MOE_DOWN_MFMA_MIN_T
#define MOE_DOWN_MFMA_MIN_T 4
#endif
#ifndef MOE_DOWN_MFMA_MIN_T_MX
#define MOE_DOWN_MFMA_MIN_T_MX 8
#endif
#ifndef MOE_DOWN_MFMA_MIN_T_WIDE
#define MOE_DOWN_MFMA_MIN_T_WIDE 12
#endif
// tokens per chunk of the MXFP4 gate/up kernel for batches of several tokens
#ifndef MOE_TT_MX
#define MOE_TT_MX 2
#endif
// largest batch the four-kernel path takes (at most 16)
#ifndef MOE_SMALL_T_MAX
#define MOE_SMALL_T_MAX 16
#endif

namespace sbk {
constexpr int TMAX = 16;
constexpr int RT = 8;            // output rows per K3 workgroup
constexpr int MAXP = TMAX * 17;  // pairs: T*K routed + T shared, K <= 16
}  // namespace sbk

// Slot table (written by the gate/up workgroups of column 0): entry j
// describes expert slot j -- the shared expert first, then the active routed
// experts in ascending order -- as SLOT_W int32: expert (-1 = shared), token
// count, TMAX pair ids (routed: slot id t*K+k; shared: T*K+t), TMAX token ids,
// then the expert's record address (two int32 at SLOT_PTR).  Entries past the
// last slot have a token count of 0.  A consumer reads its entry in one round
// trip.
constexpr int SLOT_PTR = 2 + 2 * sbk::TMAX;
constexpr int SLOT_W = SLOT_PTR + 2;

// Q8_0 of one 32-block held by 8 consecutive lanes (4 values each).
__device__ __forceinline__ uint32_t q8_quad(float4 v, float *dd_out) {
  float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  m = fmaxf(m, __shfl_xor(m, 1, 8));
  m = fmaxf(m, __shfl_xor(m, 2, 8));
  m = fmaxf(m, __shfl_xor(m, 4, 8));
  const float dd = m / 127.0f;
  const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
  auto cv = [&](float f) -> uint32_t {
    float r = roundf(f * id);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(uint8_t)(int8_t)(int)r;
  };
  *dd_out = dd;
  return cv(v.x) | (cv(v.y) << 8) | (cv(v.z) << 16) | (cv(v.w) << 24);
}

// Q8_0 of h as the down kernel reads it.  Lane jj (0..7) of a block's 8
// quantises the values k0, k0 + ks, k0 + 2 ks, k0 + 3 ks of the block and
// stores them as one word at byte `off` of the pair's row.  Natural order
// (codes 4 jj .. 4 jj + 3) for every format but int2, whose down kernel dots
// a 64-code piece field by field: there word 4 fi + j of a piece holds codes
// 16 j + fi + 4 i (i = 0..3), the bytes the dots take, so no lane has to
// rearrange them.  Codes and block scales are those of the natural order.
template <int WB>
__device__ __forceinline__ void h_word(int blk, int jj, int &k0, int &ks, int &off) {
  if constexpr (WB == 2) {
    const int fi = jj & 3, jp = jj >> 2;
    k0 = 16 * jp + fi;
    ks = 4;
    off = (blk >> 1) * 64 + (4 * fi + 2 * (blk & 1) + jp) * 4;
  } else {
    k0 = 4 * jj;
    ks = 1;
    off = blk * 32 + 4 * jj;
  }
}

// ============================================================ K1: router

// Router workgroup e (one per expert): Q8_0 of a slice of x for the expert
// kernels, then the fixed-order fp32 logit and the sigmoid score of expert e
// for every token.  Thread l < H/64 of half h owns chunk l (an fma chain
// over its 64 elements in index order) of the tokens t = h, h+2, ...
// Workgroup (x, g): experts EB x .. EB x + EB - 1 for the tokens g, g + G,
// ... (G = gridDim.y).  One CU streams only a few tens of GB/s, so with
// several tokens a workgroup's time follows the bytes it reads: all its
// tokens' inputs and its experts' weights.  EB = 2 and G = 2 halve the input
// bytes for twice the weight bytes, with the same number of workgroups.
template <int EB>
__global__ void __launch_bounds__(256) k_route_small(LayerArgs a) {
  __shared__ float part[EB][sbk::TMAX][128];
  const int e0 = blockIdx.x * EB, g = blockIdx.y, G = gridDim.y, tid = threadIdx.x;
  const int H = a.H, E = a.E, T = a.T;
  const int nt = (T - g + G - 1) / G;  // this workgroup's tokens: g + G j, j < nt
  const int half = tid >> 7, l = tid & 127;
  const int nch = H / 64;
  const bool dot = half < nt && l < nch;
  // this lane's 64 router weights of each expert and its first token's 64
  // inputs, requested before the Q8_0 work below so that all share one memory
  // round trip
  float4 wv[EB][16], xv[16];
  if (dot) {
    // ordinary loads: this one round trip is latency-bound, and non-temporal
    // loads made it slower (5.3 -> 7.7 us per decode step)
#pragma unroll
    for (int b = 0; b < EB; b++) {
      const float4 *w4 = reinterpret_cast<const float4 *>(a.wr + (size_t)(e0 + b) * H + l * 64);
#pragma unroll
      for (int k = 0; k < 16; k++) wv[b][k] = w4[k];
    }
    const float4 *x4 = reinterpret_cast<const float4 *>(a.x + (size_t)(g + G * half) * H + l * 64);
#pragma unroll
    for (int k = 0; k < 16; k++) xv[k] = x4[k];
  }
  {  // Q8_0 of a slice of x, 8 lanes per block of 32
    const int nwg = gridDim.x * G, wg = blockIdx.x * G + g;
    const int nbx = T * (H / 32);
    const int per = (nbx + nwg - 1) / nwg;
    const int b0 = wg * per, b1 = min(nbx, b0 + per);
    for (int base = b0; base < b1; base += 32) {
      const int blk = base + (tid >> 3), sub = tid & 7;
      const bool ok = blk < b1;
      const float4 v = ok ? reinterpret_cast<const float4 *>(a.x)[(size_t)blk * 8 + sub]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      float dd;
      const uint32_t packed = q8_quad(v, &dd);
      if (ok) {
        reinterpret_cast<uint32_t *>(a.q)[(size_t)blk * 8 + sub] = packed;
        if (sub == 0) a.d[blk] = dd;
      }
    }
  }
  if (dot) {
    for (int j = half; j < nt; j += 2) {
      if (j > half) {
        const float4 *x4 =
            reinterpret_cast<const float4 *>(a.x + (size_t)(g + G * j) * H + l * 64);
#pragma unroll
        for (int k = 0; k < 16; k++) xv[k] = x4[k];
      }
      // keep every load of x ahead of the chains (one memory latency, not
      // sixteen): nothing is scheduled across this point
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < EB; b++) {
        float acc = 0.0f;  // an fma chain in index order
#pragma unroll
        for (int k = 0; k < 16; k++) {
          acc = __builtin_fmaf(xv[k].x, wv[b][k].x, acc);
          acc = __builtin_fmaf(xv[k].y, wv[b][k].y, acc);
          acc = __builtin_fmaf(xv[k].z, wv[b][k].z, acc);
          acc = __builtin_fmaf(xv[k].w, wv[b][k].w, acc);
        }
        part[b][j][l] = acc;
      }
    }
  }
  __syncthreads();
  if (tid < EB * nt) {  // chunk partials added left to right
    const int b = tid / nt, j = tid % nt, t = g + G * j, e = e0 + b;
    float tot = part[b][j][0];
    for (int c = 1; c < nch; c++) tot = tot + part[b][j][c];
    const float sv = sigmoid_fixed(tot);
    a.s[(size_t)t * E + e] = sv;
    a.sb[(size_t)t * E + e] = sv + a.bias[e];
  }
}

// ============================================================ selection of one token

// The key arrays are read as ulonglong2 and ssel as float4 (16-byte LDS
// reads), so each starts on a 16-byte boundary.
struct alignas(16) SelLds {
  alignas(16) unsigned long long key[1024];   // (biased score, -index) of every expert
  alignas(16) unsigned long long fkey[1024];  // finalists: K per kept group (0 = empty)
  alignas(16) unsigned long long gkey[64];
  alignas(16) float sb[1024];                 // biased scores of the token
  alignas(16) float s[1024];                  // its unbiased scores
  alignas(16) float ssel[16];                 // unbiased scores of the picks, rank order
  unsigned long long kmask;
  int fe[1024];
  int sel[16];
};
static_assert(offsetof(SelLds, key) % 16 == 0 && offsetof(SelLds, fkey) % 16 == 0 &&
                  offsetof(SelLds, sb) % 16 == 0 && offsetof(SelLds, ssel) % 16 == 0,
              "16-byte LDS reads of the selection arrays");

// running top-2 of a sequence of values (the two largest, multiset)
__device__ __forceinline__ void top2(float v, float &m1, float &m2) {
  const float hi = fmaxf(m1, v), lo = fminf(m1, v);
  m1 = hi;
  m2 = fmaxf(m2, lo);
}

__device__ __forceinline__ unsigned long long rank_key(float v, int i) {
  return ((unsigned long long)float_key(v) << 32) | (0xFFFFFFFFu - (uint32_t)i);
}

// Selection for token t by the whole block, by ranks instead of repeated
// argmax: with key = (score, -index) (all distinct), an item is among the
// best n exactly when fewer than n items have a larger key, and its rank is
// its position in the descending order; this is the same set and order as
// picking the maximum n times with ties to the lower index.
__device__ void select_token(const LayerArgs &a, SelLds &sm, int t) {
  const int E = a.E, G = a.G, gs = E / G, K = a.K;
  for (int e = threadIdx.x; e < E; e += 256) {
    const float v = a.sb[(size_t)t * E + e];
    sm.sb[e] = v;
    sm.s[e] = a.s[(size_t)t * E + e];
    sm.key[e] = rank_key(v, e);
  }
  __syncthreads();
  if (threadIdx.x < G) {  // group score: sum of the two largest biased scores
    const int g = threadIdx.x;
    float m1 = -INFINITY, m2 = -INFINITY;
    const float *p = sm.sb + g * gs;
    if ((gs & 15) == 0) {  // 4 independent 16-byte LDS reads per step
      for (int e = 0; e < gs; e += 16) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) v[u] = *reinterpret_cast<const float4 *>(p + e + 4 * u);
#pragma unroll
        for (int u = 0; u < 4; u++) {
          top2(v[u].x, m1, m2);
          top2(v[u].y, m1, m2);
          top2(v[u].z, m1, m2);
          top2(v[u].w, m1, m2);
        }
      }
    } else {
      for (int e = 0; e < gs; e++) top2(p[e], m1, m2);
    }
    sm.gkey[g] = rank_key(m1 + m2, g);
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // kept groups as a bitmask (G <= 64)
    bool kept = false;
    if (threadIdx.x < G) {
      const unsigned long long mine = sm.gkey[threadIdx.x];
      int r = 0;
      for (int g = 0; g < G; g++) r += sm.gkey[g] > mine;
      kept = r < a.TG;
    }
    const unsigned long long m = __ballot(kept);
    if (threadIdx.x == 0) sm.kmask = m;
  }
  const int F = a.TG * K;  // finalist slots: K per kept group
  for (int f = threadIdx.x; f < F; f += 256) sm.fkey[f] = 0ull;
  __syncthreads();
  // stage A: rank within the group; a global top-K item is in its group's
  // top-K, so each kept group hands its best K to slots j*K .. j*K+K-1
  const unsigned long long kmask = sm.kmask;
  for (int e = threadIdx.x; e < E; e += 256) {
    const int g = e / gs;
    if (!((kmask >> g) & 1ull)) continue;
    const unsigned long long mine = sm.key[e];
    const unsigned long long *kk = sm.key + g * gs;
    int r = 0;
    if ((gs & 15) == 0) {  // 8 independent 16-byte LDS reads per step
      for (int i = 0; i < gs; i += 16) {
        ulonglong2 v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = *reinterpret_cast<const ulonglong2 *>(kk + i + 2 * u);
#pragma unroll
        for (int u = 0; u < 8; u++) r += (v[u].x > mine) + (v[u].y > mine);
      }
    } else {
      for (int i = 0; i < gs; i++) r += kk[i] > mine;
    }
    if (r < K) {
      const int j = __popcll(kmask & ((1ull << g) - 1ull));
      sm.fkey[j * K + r] = mine;
      sm.fe[j * K + r] = e;
    }
  }
  __syncthreads();
  // stage B: rank among the finalists = rank among all candidates
  for (int f = threadIdx.x; f < F; f += 256) {
    const unsigned long long mine = sm.fkey[f];
    if (mine == 0ull) continue;
    int r = 0;
    int i = 0;
    for (; i + 16 <= F; i += 16) {
      ulonglong2 v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) v[u] = *reinterpret_cast<const ulonglong2 *>(sm.fkey + i + 2 * u);
#pragma unroll
      for (int u = 0; u < 8; u++) r += (v[u].x > mine) + (v[u].y > mine);
    }
    for (; i < F; i++) r += sm.fkey[i] > mine;
    if (r < K) {
      sm.sel[r] = sm.fe[f];
      sm.ssel[r] = sm.s[sm.fe[f]];
    }
  }
  __syncthreads();
  if (threadIdx.x < K) {  // weights: unbiased scores over their sum in rank order
    float sv[16];
#pragma unroll
    for (int k = 0; k < 16; k += 4) {  // four 16-byte reads, one round trip
      const float4 v4 = *reinterpret_cast<const float4 *>(sm.ssel + k);
      sv[k] = v4.x;
      sv[k + 1] = v4.y;
      sv[k + 2] = v4.z;
      sv[k + 3] = v4.w;
    }
    float S = sv[0];
#pragma unroll
    for (int k = 1; k < 16; k++) S = (k < K) ? S + sv[k] : S;
    float Sk;
    const int n = top_p_keep(sv, K, S, a.top_p, &Sk);  // n = K unless top-p cuts
    const bool keep = (int)threadIdx.x < n;
    a.idx[t * K + threadIdx.x] = keep ? sm.sel[threadIdx.x] : -1;
    a.w[t * K + threadIdx.x] = keep ? (sm.ssel[threadIdx.x] / Sk) * a.scale : 0.0f;
  }
}


// ============================================================ operands

template <int WB>
struct Act;
template <>
struct Act<4> {
  QBlock q;
  float d;  // block scale / 16 (the int4 dot returns 16 x the block dot)
};
template <>
struct Act<2> {
  int f[4][4];
  float da, db;  // scales / 64 of the two blocks of a 64-code piece
};

template <>
struct Act<8> {
  int q[4];  // 16 activations (half a Q8_0 block), natural order
  float d;   // the block's scale
};
template <>
struct Act<WB_MX> {
  QBlock q;
  float d;  // block scale / 2 (the MXFP4 dot returns 2 x the block dot)
};
template <>
struct Act<WB_F8> {  // as int8: 16 activations (half a Q8_0 block)
  int q[4];
  float d;
};

// One 16-byte weight piece; for MXFP4 also its block's scale.
template <int WB>
struct WP {
  uint4 w;
};
template <>
struct WP<WB_MX> {
  uint4 w;
  float s;
};
template <>
struct WP<WB_F8> {
  uint4 w;
  float s;  // the 128x128 block's scale
};

// Piece p of a weight row (scl: the row's E8M0 bytes for MXFP4, the fp32
// scales of the row's 128-row block for FP8 (8 pieces per scale); with
// SCALE false the scale is filled in later).
template <int WB, bool SCALE = true>
__device__ __forceinline__ WP<WB> load_wp(const uint8_t *row, const uint8_t *scl, int p,
                                          bool ok) {
  WP<WB> r;
  r.w = ok ? gload<uint4>(row, (size_t)p * 16) : make_uint4(0, 0, 0, 0);
  if constexpr (WB == WB_MX) r.s = (SCALE && ok) ? e8m0_float(gload<uint8_t>(scl, p)) : 0.0f;
  if constexpr (WB == WB_F8) r.s = (SCALE && ok) ? gload<float>(scl, 4 * (size_t)(p >> 3)) : 0.0f;
  return r;
}

// A weight piece as loaded, for kernels that keep several loads in flight:
// read unconditionally from a valid address and masked where it is used, so
// that no branch holds the load (a branch around a load makes the compiler
// wait for every load issued before it).
template <int WB>
struct WRaw {
  uint4 w;
};
template <>
struct WRaw<WB_MX> {
  uint4 w;
  uint32_t sb;  // the block's E8M0 byte
};
template <>
struct WRaw<WB_F8> {
  uint4 w;
  float s;
};
template <int WB, bool SCALE = true>
__device__ __forceinline__ WRaw<WB> load_wraw(const uint8_t *row, const uint8_t *scl, int p) {
  WRaw<WB> r;
  r.w = gload_stream(row, (size_t)p * 16);
  if constexpr (WB == WB_MX) r.sb = SCALE ? gload<uint8_t>(scl, p) : 0u;
  if constexpr (WB == WB_F8) r.s = SCALE ? gload<float>(scl, 4 * (size_t)(p >> 3)) : 0.0f;
  return r;
}
// The piece, or zeros when !ok.
template <int WB>
__device__ __forceinline__ WP<WB> cook_wp(const WRaw<WB> &r, bool ok) {
  WP<WB> o;
  o.w = ok ? r.w : make_uint4(0, 0, 0, 0);
  if constexpr (WB == WB_MX) o.s = ok ? e8m0_float(r.sb) : 0.0f;
  if constexpr (WB == WB_F8) o.s = ok ? r.s : 0.0f;
  return o;
}

// An activation piece as loaded: its bytes and block scale(s), not yet
// rearranged, so that a load can stay in flight until the piece is used.
template <int WB>
struct ActRaw {
  uint4 x[byte_codes(WB) ? 1 : WB == 2 ? 4 : 2];
  float d0, d1;
};

// Piece p of a Q8_0 row (q, d); zeros when !ok.
template <int WB>
__device__ __forceinline__ ActRaw<WB> load_act_raw(const int8_t *q, const float *d, int p,
                                                   bool ok) {
  constexpr int NX = byte_codes(WB) ? 1 : WB == 2 ? 4 : 2;
  ActRaw<WB> r;
#pragma unroll
  for (int j = 0; j < NX; j++) r.x[j] = make_uint4(0, 0, 0, 0);
  r.d0 = r.d1 = 0.0f;
  if (ok) {
    const uint4 *qp = reinterpret_cast<const uint4 *>(q + 16 * NX * p);
#pragma unroll
    for (int j = 0; j < NX; j++) r.x[j] = qp[j];
    if constexpr (byte_codes(WB)) {
      r.d0 = d[p >> 1];
    } else if constexpr (WB == 2) {
      r.d0 = d[2 * p];
      r.d1 = d[2 * p + 1];
    } else {
      r.d0 = d[p];
    }
  }
  return r;
}

// The loaded piece in the layout the dot products take.
template <int WB>
__device__ __forceinline__ Act<WB> cook_act(const ActRaw<WB> &r);
template <>
__device__ __forceinline__ Act<8> cook_act<8>(const ActRaw<8> &r) {
  Act<8> o;
  o.q[0] = (int)r.x[0].x;
  o.q[1] = (int)r.x[0].y;
  o.q[2] = (int)r.x[0].z;
  o.q[3] = (int)r.x[0].w;
  o.d = r.d0;
  return o;
}
template <>
__device__ __forceinline__ Act<WB_F8> cook_act<WB_F8>(const ActRaw<WB_F8> &r) {
  Act<WB_F8> o;
  o.q[0] = (int)r.x[0].x;
  o.q[1] = (int)r.x[0].y;
  o.q[2] = (int)r.x[0].z;
  o.q[3] = (int)r.x[0].w;
  o.d = r.d0;
  return o;
}
template <>
__device__ __forceinline__ Act<4> cook_act<4>(const ActRaw<4> &r) {
  Act<4> o;
  o.q = split_block(r.x[0], r.x[1]);
  o.d = r.d0 * (1.0f / 16.0f);
  return o;
}
template <>
__device__ __forceinline__ Act<WB_MX> cook_act<WB_MX>(const ActRaw<WB_MX> &r) {
  Act<WB_MX> o;
  o.q = split_block(r.x[0], r.x[1]);
  o.d = r.d0 * 0.5f;
  return o;
}
template <>
__device__ __forceinline__ Act<2> cook_act<2>(const ActRaw<2> &r) {
  Act<2> o;
#pragma unroll
  for (int j = 0; j < 4; j++) {
#pragma unroll
    for (int fi = 0; fi < 4; fi++) {
      const uint32_t sel = (uint32_t)(fi | ((4 + fi) << 8)) | 0x0C0C0000u;
      const uint32_t a01 = __builtin_amdgcn_perm(r.x[j].y, r.x[j].x, sel);
      const uint32_t a23 = __builtin_amdgcn_perm(r.x[j].w, r.x[j].z, sel);
      o.f[fi][j] = (int)__builtin_amdgcn_perm(a23, a01, 0x05040100u);
    }
  }
  o.da = r.d0 * (1.0f / 64.0f);
  o.db = r.d1 * (1.0f / 64.0f);
  return o;
}

// A piece of Q8_0(h) as the down kernel loads it (laid out by h_word): int2
// pieces are already in field order, the others as cook_act takes them.
template <int WB>
__device__ __forceinline__ Act<WB> cook_act_h(const ActRaw<WB> &r) {
  if constexpr (WB == 2) {
    Act<2> o;
#pragma unroll
    for (int fi = 0; fi < 4; fi++) {
      o.f[fi][0] = (int)r.x[fi].x;
      o.f[fi][1] = (int)r.x[fi].y;
      o.f[fi][2] = (int)r.x[fi].z;
      o.f[fi][3] = (int)r.x[fi].w;
    }
    o.da = r.d0 * (1.0f / 64.0f);
    o.db = r.d1 * (1.0f / 64.0f);
    return o;
  } else {
    return cook_act<WB>(r);
  }
}

template <int WB>
__device__ __forceinline__ void load_act(const int8_t *q, const float *d, int p, bool ok,
                                         Act<WB> &o) {
  o = cook_act<WB>(load_act_raw<WB>(q, d, p, ok));
}

// The exact integer dot(s) of one 16-byte weight piece with one token's
// activations, as the lanes compute them: int4 gives 16 x the block dot (its
// codes enter as 16 x code), int2 64 x the dots of its two 32-code blocks,
// int8 the dot of half a block (16 codes), MXFP4 the block dot of the doubled
// FP4 values, FP8 the dot of half a block with the codes as 512 x value.
// Every float sum below is built from these.
template <int WB>
struct PDots {
  int v[WB == 2 ? 2 : 1];
};

template <int WB>
__device__ __forceinline__ PDots<WB> piece_idot(const WP<WB> &p, const Act<WB> &a);
template <>
__device__ __forceinline__ PDots<WB_MX> piece_idot<WB_MX>(const WP<WB_MX> &p, const Act<WB_MX> &a) {
  return PDots<WB_MX>{{dot_mx_block(p.w, a.q)}};
}
template <>
__device__ __forceinline__ PDots<8> piece_idot<8>(const WP<8> &p, const Act<8> &a) {
  const uint4 w = p.w;
  int acc = sdot4((int)w.x, a.q[0], 0);  // 16 int8 codes: exact, |acc| < 2^19
  acc = sdot4((int)w.y, a.q[1], acc);
  acc = sdot4((int)w.z, a.q[2], acc);
  acc = sdot4((int)w.w, a.q[3], acc);
  return PDots<8>{{acc}};
}
template <>
__device__ __forceinline__ PDots<WB_F8> piece_idot<WB_F8>(const WP<WB_F8> &p,
                                                          const Act<WB_F8> &a) {
  int acc = dot_fp8_word(p.w.x, (uint32_t)a.q[0], 0);
  acc = dot_fp8_word(p.w.y, (uint32_t)a.q[1], acc);
  acc = dot_fp8_word(p.w.z, (uint32_t)a.q[2], acc);
  acc = dot_fp8_word(p.w.w, (uint32_t)a.q[3], acc);
  return PDots<WB_F8>{{acc}};
}
template <>
__device__ __forceinline__ PDots<4> piece_idot<4>(const WP<4> &p, const Act<4> &a) {
  return PDots<4>{{dot_int4_block16(p.w, a.q)}};
}
template <>
__device__ __forceinline__ PDots<2> piece_idot<2>(const WP<2> &p, const Act<2> &a) {
  const uint4 w = p.w;
  int x = 0, y = 0;
#pragma unroll
  for (int fi = 0; fi < 4; fi++) {
    x = sdot4(int2_field64(w.x, fi), a.f[fi][0], x);
    x = sdot4(int2_field64(w.y, fi), a.f[fi][1], x);
    y = sdot4(int2_field64(w.z, fi), a.f[fi][2], y);
    y = sdot4(int2_field64(w.w, fi), a.f[fi][3], y);
  }
  return PDots<2>{{x, y}};
}

// sum_b d_b * P_b of the piece from its integer dot(s); ws is the MXFP4 or
// FP8 block scale (unused by the other formats).
template <int WB>
__device__ __forceinline__ float pdots_value(const PDots<WB> &r, const Act<WB> &a, float ws) {
  if constexpr (WB == 2) return fmaf((float)r.v[0], a.da, (float)r.v[1] * a.db);
  else if constexpr (WB == WB_MX || WB == WB_F8) return (float)r.v[0] * (a.d * ws);
  else return (float)r.v[0] * a.d;
}

// sum_b d_b * P_b of one 16-byte weight piece against one token
template <int WB>
__device__ __forceinline__ float piece_dot(const WP<WB> &p, const Act<WB> &a) {
  float ws = 1.0f;
  if constexpr (WB == WB_MX || WB == WB_F8) ws = p.s;
  return pdots_value<WB>(piece_idot<WB>(p, a), a, ws);
}

// A weight piece made ready for several tokens: MXFP4 codes turned into
// int8 lanes once (the lookup costs more than the dots); other formats as
// loaded.
template <int WB>
struct WReady {
  WP<WB> p;
};
template <>
struct WReady<WB_MX> {
  int l[8];  // even / odd lanes of words 0..3: 2 x the FP4 values
  float s;
};
template <int WB>
__device__ __forceinline__ WReady<WB> ready(const WP<WB> &p) {
  return WReady<WB>{p};
}
template <>
__device__ __forceinline__ WReady<WB_MX> ready<WB_MX>(const WP<WB_MX> &p) {
  WReady<WB_MX> r;
  const uint32_t w[4] = {p.w.x, p.w.y, p.w.z, p.w.w};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    r.l[2 * j] = mx_lanes(w[j], 0);
    r.l[2 * j + 1] = mx_lanes(w[j], 4);
  }
  r.s = p.s;
  return r;
}
template <int WB>
__device__ __forceinline__ PDots<WB> ready_idot(const WReady<WB> &w, const Act<WB> &a) {
  if constexpr (WB == WB_MX) {
    int acc = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      acc = sdot4(w.l[2 * j], a.q.ev[j], acc);
      acc = sdot4(w.l[2 * j + 1], a.q.od[j], acc);
    }
    return PDots<WB_MX>{{acc}};
  } else {
    return piece_idot<WB>(w.p, a);
  }
}
template <int WB>
__device__ __forceinline__ float ready_scale(const WReady<WB> &w) {
  if constexpr (WB == WB_MX) return w.s;
  else if constexpr (WB == WB_F8) return w.p.s;
  else return 1.0f;
}
// At the top of a token loop over weights held in registers: FP8 codes are
// marked changed, so that they are converted where each token uses them
// rather than all at once before the loop (16 integers per piece: 256
// registers, then spills).
template <int WB>
__device__ __forceinline__ void fresh_codes(uint4 &w) {
  if constexpr (WB == WB_F8) opaque_words(w);
}

template <int WB>
__device__ __forceinline__ float ready_dot(const WReady<WB> &w, const Act<WB> &a) {
  return pdots_value<WB>(ready_idot<WB>(w, a), a, ready_scale<WB>(w));
}

// Debug dumps (moe_layer_debug): the block dot(s) of piece p of a row (p
// counted along the whole row) into dots [pair][R rows][nblk blocks], as
// reported: int4 >> 4, int2 >> 6 (two blocks), MXFP4 as is, and for int8
// and FP8 the sum of the two half-block dots, which sit in adjacent lanes
// (pieces 2b and 2b + 1; the even lane stores).  Every lane of the wave calls it
// (the int8 exchange is a wave operation); ok masks the store.
template <int WB>
__device__ __forceinline__ void dump_pdots(int32_t *dots, const PDots<WB> &r, int pair, int row,
                                           int R, int nblk, int p, bool ok) {
  const size_t base = ((size_t)pair * R + row) * nblk;
  if constexpr (byte_codes(WB)) {
    const int s = r.v[0] + __shfl_xor(r.v[0], 1);
    if (ok && (p & 1) == 0) dots[base + (p >> 1)] = s;
  } else if constexpr (WB == 2) {
    if (ok) {
      dots[base + 2 * p] = r.v[0] >> 6;
      dots[base + 2 * p + 1] = r.v[1] >> 6;
    }
  } else if constexpr (WB == 4) {
    if (ok) dots[base + p] = r.v[0] >> 4;
  } else {
    if (ok) dots[base + p] = r.v[0];
  }
}

// Debug dump of one Q8_0 word of h as q8_quad packed it: the codes of
// values k0, k0 + ks, k0 + 2 ks, k0 + 3 ks of block blk, in natural order.
__device__ __forceinline__ void dump_q8_word(int8_t *q_h, float *d_h, int pair, int I, int blk,
                                             int k0, int ks, uint32_t packed, float dd,
                                             bool first) {
  if (q_h) {
#pragma unroll
    for (int m = 0; m < 4; m++)
      q_h[(size_t)pair * I + blk * 32 + k0 + m * ks] = (int8_t)(packed >> (8 * m));
  }
  if (d_h && first) d_h[(size_t)pair * (I / 32) + blk] = dd;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 32 rows of h (rows 32 blk ..) for one expert and n_tok tokens.  KS = 1:
// wave wv streams rows 8wv .. 8wv+7 whole; KS = 2 (long int8 rows): waves
// wv and wv+2 stream rows 16(wv&1) .. +15, each over one half of the hidden
// dimension, and the halves are added in LDS.  Rows go in batches of RB (a
// gate and an up row each), double-buffered.  Activations of token i: Q8_0
// codes/scales at qrow(i)/drow(i).  h goes to LDS; each token's 32 values
// become one Q8_0 block of q_h.
// MXFP4: the block scales of the workgroup's 32 gate and 32 up rows, staged
// once with 16-byte loads (one byte load per piece would double the load
// instructions of the weight stream): msc[gate, up][32 rows][H/32 <= 256]
constexpr int GU_MSC = 32 * 256;
// FP8: the 32 rows lie in one 128-row block, whose H/128 <= 64 fp32 scales
// of gate and of up are staged: msc as float [gate, up][F8_MSC]
constexpr int F8_MSC = 64;
template <int WB>
constexpr int gu_msc_bytes() {
  return WB == WB_MX ? 2 * GU_MSC : WB == WB_F8 ? 2 * F8_MSC * 4 : 16;
}
// Stage the FP8 scales of rows blk*32.. (every thread calls it).
__device__ __forceinline__ void stage_f8_scales(uint8_t *msc, const uint8_t *tail, int H, int I,
                                                int blk) {
  float *fs = reinterpret_cast<float *>(msc);
  const int nsb = H / 128;
  const size_t gs = 4 * (size_t)((blk * 32) / 128) * nsb;
  const size_t us = 4 * (size_t)(I / 128) * nsb + gs;
  for (int i = threadIdx.x; i < 2 * nsb; i += 256)
    fs[i < nsb ? i : F8_MSC + i - nsb] = gload<float>(tail, i < nsb ? gs + 4 * i : us + 4 * (i - nsb));
}

template <int WB, int TT, int NPL, int RB, int KS, bool DBG, class QRow, class DRow>
__device__ void gate_up_rows(const LayerArgs &a, float (*hb)[32], uint8_t *msc,
                             const uint8_t *blob, int blk, int n_tok, const int *pairs, QRow qrow,
                             DRow drow) {
  static_assert(KS == 1 || KS == 2, "K split");
  static_assert(WB != WB_MX || KS == 1, "MXFP4 rows fit one wave");
  __shared__ float part[KS][TT][32][2];  // KS = 2: scaled half sums (gate, up)
  constexpr int MSC = GU_MSC;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I;
  constexpr int RW = 8 * KS;  // rows per wave
  const int khalf = wv / (4 / KS), wr = wv % (4 / KS);
  const int np_all = H / (128 / code_bits<WB>()), np_half = (np_all + KS - 1) / KS;
  const int p0 = khalf * np_half, npieces = min(np_all, p0 + np_half);
  const size_t row_b = (size_t)H * code_bits<WB>() / 8;
  const uint8_t *gate = blob;
  const uint8_t *up = blob + (size_t)I * row_b;
  const uint8_t *tail = blob + 3 * (size_t)I * row_b;  // row scales, or MXFP4 block scales
  const int nblk = H / 32;
  const uint8_t *gsc = tail, *usc = tail + (size_t)I * nblk;  // MXFP4
  const int rbase = blk * 32 + wr * RW;
  // row scales of the wave's rows: lane l < RW gate row l, RW <= l < 2 RW up row l - RW
  const float sc = lane >= 2 * RW ? 0.0f
                   : WB == WB_MX ? 1.0f
                   : WB == WB_F8 ? 1.0f / 512.0f  // the codes enter as 512 x value
                                 : gload<float>(tail, 4 * (size_t)((lane < RW ? 0 : I) + rbase +
                                                                   lane % RW));
  constexpr int NB = RW / RB;
  for (int c0 = 0; c0 < n_tok; c0 += TT) {
    // two buffers: batch bt+1 is in flight while batch bt is computed.  Every
    // load is unconditional (lanes past the row read its first piece and are
    // masked where the piece is used), so that the compiler can wait for one
    // batch while the next stays in flight.
    WRaw<WB> wb[2][RB][2][NPL];  // [buffer][row of batch][gate, up][piece]
    auto load_batch = [&](WRaw<WB> (&dst)[RB][2][NPL], int bt) {
#pragma unroll
      for (int rr = 0; rr < RB; rr++) {
        const int r = rbase + bt * RB + rr;
#pragma unroll
        for (int i = 0; i < NPL; i++) {
          const int p = p0 + lane + 64 * i;
          const int pc = p < npieces ? p : p0;
          dst[rr][0][i] = load_wraw<WB, false>(gate + (size_t)r * row_b, nullptr, pc);
          dst[rr][1][i] = load_wraw<WB, false>(up + (size_t)r * row_b, nullptr, pc);
        }
      }
    };
    // the activations first (cache hits), then the first batch: the
    // activations are rearranged while that batch is in flight
    ActRaw<WB> araw[NPL][TT];
#pragma unroll
    for (int t = 0; t < TT; t++) {
      const int tok = c0 + t < n_tok ? c0 + t : c0;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = p0 + lane + 64 * i;
        araw[i][t] = load_act_raw<WB>(qrow(tok), drow(tok), p < npieces ? p : p0, true);
      }
    }
    load_batch(wb[0], 0);
    if constexpr (WB == WB_MX) {
      if (c0 == 0) {  // rows blk*32 .. +31 of each matrix: 32 * nblk contiguous bytes
        const int n16 = 32 * nblk / 16;
        for (int i = threadIdx.x; i < 2 * n16; i += 256) {
          const int m = i / n16, o = (i % n16) * 16;
          *reinterpret_cast<uint4 *>(msc + m * MSC + o) =
              gload<uint4>(m ? usc : gsc, (size_t)blk * 32 * nblk + o);
        }
        __syncthreads();
      }
    }
    if constexpr (WB == WB_F8) {
      if (c0 == 0) {
        stage_f8_scales(msc, tail, H, I, blk);
        __syncthreads();
      }
    }
    // lanes past the row: zero activations (their weight pieces, read from
    // the row's first piece, then add exact zeros)
    Act<WB> act[NPL][TT];
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      const bool ok = p0 + lane + 64 * i < npieces;
#pragma unroll
      for (int t = 0; t < TT; t++) act[i][t] = cook_act<WB>(ok ? araw[i][t] : ActRaw<WB>{});
    }
#pragma unroll
    for (int bt = 0; bt < NB; bt++) {
      if (bt + 1 < NB) load_batch(wb[(bt + 1) & 1], bt + 1);
      // the next batch's loads go out before this batch is reduced
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rr = 0; rr < RB; rr++) {
        const int rl = bt * RB + rr;  // row within the wave's RW
        WP<WB> wg[NPL], wu[NPL];
#pragma unroll
        for (int i = 0; i < NPL; i++) {
          const bool ok = p0 + lane + 64 * i < npieces;
          wg[i] = cook_wp<WB>(wb[bt & 1][rr][0][i], true);
          wu[i] = cook_wp<WB>(wb[bt & 1][rr][1][i], true);
          if constexpr (WB == WB_MX) {
            const int o = (wr * RW + rl) * nblk + lane + 64 * i;
            wg[i].s = ok ? e8m0_float(msc[o]) : 0.0f;
            wu[i].s = ok ? e8m0_float(msc[MSC + o]) : 0.0f;
          }
          if constexpr (WB == WB_F8) {  // 8 pieces per 128-column block
            const int o = (ok ? p0 + lane + 64 * i : p0) >> 3;
            const float *fs = reinterpret_cast<const float *>(msc);
            wg[i].s = ok ? fs[o] : 0.0f;
            wu[i].s = ok ? fs[F8_MSC + o] : 0.0f;
          }
        }
        float g[TT], u[TT];
#pragma unroll
        for (int t = 0; t < TT; t++) g[t] = u[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; i++) {
          const WReady<WB> rg = ready<WB>(wg[i]);
          const WReady<WB> ru = ready<WB>(wu[i]);
#pragma unroll
          for (int t = 0; t < TT; t++) {
            const PDots<WB> dg = ready_idot<WB>(rg, act[i][t]);
            g[t] += pdots_value<WB>(dg, act[i][t], ready_scale<WB>(rg));
            const PDots<WB> du = ready_idot<WB>(ru, act[i][t]);
            u[t] += pdots_value<WB>(du, act[i][t], ready_scale<WB>(ru));
            if constexpr (DBG) {
              const int p = p0 + lane + 64 * i;
              const bool ok = p < npieces && c0 + t < n_tok;
              const int pr = pairs[min(c0 + t, n_tok - 1)];
              if (a.dbg.ffn.gate_dots)
                dump_pdots<WB>(a.dbg.ffn.gate_dots, dg, pr, rbase + rl, I, H / 32, p, ok);
              if (a.dbg.ffn.up_dots)
                dump_pdots<WB>(a.dbg.ffn.up_dots, du, pr, rbase + rl, I, H / 32, p, ok);
            }
          }
        }
        const float sg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), rl));
        const float su = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), RW + rl));
#pragma unroll
        for (int t = 0; t < TT; t++) {
          const float gv = sg * wave_sum(g[t]);
          const float uv = su * wave_sum(u[t]);
          if (lane == 0) {
            if constexpr (KS == 1) {
              hb[t][wv * 8 + rl] = silu(gv) * uv;
              if (DBG && a.dbg.ffn.h && c0 + t < n_tok)
                a.dbg.ffn.h[(size_t)pairs[c0 + t] * I + blk * 32 + wv * 8 + rl] = silu(gv) * uv;
            } else {
              part[khalf][t][wr * RW + rl][0] = gv;
              part[khalf][t][wr * RW + rl][1] = uv;
            }
          }
        }
      }
    }
    if constexpr (KS == 2) {
      __syncthreads();
      if (threadIdx.x < TT * 32) {
        const int t = threadIdx.x >> 5, r = threadIdx.x & 31;
        hb[t][r] = silu(part[0][t][r][0] + part[1][t][r][0]) *
                   (part[0][t][r][1] + part[1][t][r][1]);
        if (DBG && a.dbg.ffn.h && c0 + t < n_tok)
          a.dbg.ffn.h[(size_t)pairs[c0 + t] * I + blk * 32 + r] = hb[t][r];
      }
    }
    __syncthreads();
    if (threadIdx.x < TT * 8) {  // Q8_0 of each token's 32 h values
      const int t = threadIdx.x >> 3, j = threadIdx.x & 7;
      int k0, ks, off;
      h_word<WB>(blk, j, k0, ks, off);
      const float4 v = make_float4(hb[t][k0], hb[t][k0 + ks], hb[t][k0 + 2 * ks],
                                   hb[t][k0 + 3 * ks]);
      float dd;
      const uint32_t packed = q8_quad(v, &dd);
      if (c0 + t < n_tok) {
        const int pair = min(max(pairs[c0 + t], 0), a.T * (a.K + a.n_shared) - 1);
        *reinterpret_cast<uint32_t *>(a.qh + (size_t)pair * I + off) = packed;
        if (j == 0) a.dh[(size_t)pair * (I / 32) + blk] = dd;
        if (DBG) dump_q8_word(a.dbg.ffn.q_h, a.dbg.ffn.d_h, pair, I, blk, k0, ks, packed, dd, j == 0);
      }
    }
    __syncthreads();
  }
}

// A cooked activation piece as words: NQ 16-byte quads of codes, then NS
// scales (the member order of every Act<WB>).
template <int WB>
struct ActWords {
  static constexpr int N = sizeof(Act<WB>) / 4;
  static constexpr int NQ = byte_codes(WB) ? 1 : WB == 2 ? 4 : 2;
  static constexpr int NS = N - 4 * NQ;
};

// Tokens staged at a time by gate_up_rows_lds: up to 8, in at most 48 KB
// (a staged token holds KS NPL 64 pieces: the whole row)
constexpr int GU_ACT_LDS = 48 * 1024;
template <int WB, int TT, int NPL, int KS>
constexpr int gu_stage_tokens() {
  const int fit = GU_ACT_LDS / (KS * NPL * 64 * (int)sizeof(Act<WB>));
  return (fit < 8 ? fit : 8) / TT * TT;
}

// gate_up_rows for a slot with more tokens than one chunk: the slot's
// activations, cooked, are staged in LDS up to SG tokens at a time and every
// row is streamed once for all of them, its chunks of TT tokens read from LDS
// (from registers, each chunk would stream the rows again).  With KS = 2 a
// wave takes its half of each staged row, and the pieces past its half get
// zero weights.  Sums per token are those of gate_up_rows, in the same order.
template <int WB, int TT, int NPL, int KS, bool DBG, class QRow, class DRow>
__device__ void gate_up_rows_lds(const LayerArgs &a, uint8_t *msc, const uint8_t *blob, int blk,
                                 int n_tok, const int *pairs, QRow qrow, DRow drow) {
  static_assert(KS == 1 || KS == 2, "K split");
  static_assert(WB != WB_MX || KS == 1, "MXFP4 rows fit one wave");
  using AW = ActWords<WB>;
  constexpr int P = KS * NPL * 64;  // pieces per staged token (zeros past the row)
  constexpr int SG = gu_stage_tokens<WB, TT, NPL, KS>();
  static_assert(SG >= 2 * TT, "at least two chunks staged");
  static_assert(sizeof(Act<WB>) == 4 * (4 * AW::NQ + AW::NS), "Act<WB> as words");
  __shared__ __align__(16) uint4 aq[SG * AW::NQ * P];  // [token][quad][piece]
  __shared__ float as[SG * AW::NS * P];                // [token][scale][piece]
  __shared__ float hbs[SG][32];
  __shared__ float part[KS == 2 ? 2 : 1][KS == 2 ? SG : 1][32][2];  // KS = 2: half sums
  constexpr int MSC = GU_MSC;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I;
  constexpr int RW = 8 * KS;  // rows per wave, one per batch
  const int khalf = wv / (4 / KS), wr = wv % (4 / KS);
  const int npieces = H / (128 / code_bits<WB>());
  const int np_half = (npieces + KS - 1) / KS;
  const int p0 = khalf * np_half, pend = min(npieces, p0 + np_half);
  const size_t row_b = (size_t)H * code_bits<WB>() / 8;
  const uint8_t *gate = blob;
  const uint8_t *up = blob + (size_t)I * row_b;
  const uint8_t *tail = blob + 3 * (size_t)I * row_b;
  const int nblk = H / 32;
  const uint8_t *gsc = tail, *usc = tail + (size_t)I * nblk;  // MXFP4
  const int rbase = blk * 32 + wr * RW;
  const float sc = lane >= 2 * RW ? 0.0f
                   : WB == WB_MX ? 1.0f
                   : WB == WB_F8 ? 1.0f / 512.0f  // the codes enter as 512 x value
                                 : gload<float>(tail, 4 * (size_t)((lane < RW ? 0 : I) + rbase +
                                                                   lane % RW));
  auto load_row = [&](WRaw<WB> (&dst)[2][NPL], int rl) {
    const int r = rbase + rl;
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      const int p = p0 + lane + 64 * i;
      const int pc = p < pend ? p : p0;
      dst[0][i] = load_wraw<WB, false>(gate + (size_t)r * row_b, nullptr, pc);
      dst[1][i] = load_wraw<WB, false>(up + (size_t)r * row_b, nullptr, pc);
    }
  };
  if constexpr (WB == WB_MX) {  // block scales of the 32 gate and up rows
    const int n16 = 32 * nblk / 16;
    for (int i = tid; i < 2 * n16; i += 256) {
      const int m = i / n16, o = (i % n16) * 16;
      *reinterpret_cast<uint4 *>(msc + m * MSC + o) =
          gload<uint4>(m ? usc : gsc, (size_t)blk * 32 * nblk + o);
    }
  }
  if constexpr (WB == WB_F8) stage_f8_scales(msc, tail, H, I, blk);  // read after a barrier below
  for (int g0 = 0; g0 < n_tok; g0 += SG) {
    const int ng = min(SG, n_tok - g0);
    WRaw<WB> wb[2][2][NPL];  // [buffer][gate, up][piece]
    load_row(wb[0], 0);
    // the group's activations: every load unconditional (clamped items
    // repeat the last one and store the same values again)
    constexpr int MI = (SG * P + 255) / 256;
    const int nit = ng * P;
    ActRaw<WB> raw[MI];
#pragma unroll
    for (int k = 0; k < MI; k++) {
      const int it = min(tid + 256 * k, nit - 1);
      const int tok = it / P, p = it % P;
      raw[k] = load_act_raw<WB>(qrow(g0 + tok), drow(g0 + tok), p < npieces ? p : 0, true);
    }
    __syncthreads();  // the previous group is done with the staging
#pragma unroll
    for (int k = 0; k < MI; k++) {
      const int it = min(tid + 256 * k, nit - 1);
      const int tok = it / P, p = it % P;
      const Act<WB> c = cook_act<WB>(p < npieces ? raw[k] : ActRaw<WB>{});
      uint32_t w[AW::N];
      __builtin_memcpy(w, &c, sizeof(c));
#pragma unroll
      for (int q = 0; q < AW::NQ; q++)
        aq[(tok * AW::NQ + q) * P + p] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
#pragma unroll
      for (int j = 0; j < AW::NS; j++) as[(tok * AW::NS + j) * P + p] = __uint_as_float(w[4 * AW::NQ + j]);
    }
    __syncthreads();
#pragma unroll
    for (int rl = 0; rl < RW; rl++) {
      if (rl + 1 < RW) load_row(wb[(rl + 1) & 1], rl + 1);
      // the next row's loads go out before this one is reduced
      __builtin_amdgcn_sched_barrier(0);
      WReady<WB> rg[NPL], ru[NPL];
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        // past the wave's pieces: the staged activations are zeros past the
        // row; with KS = 2 the other half's, so the weights are zeroed there
        const bool ok = p0 + lane + 64 * i < pend;
        WP<WB> wg = cook_wp<WB>(wb[rl & 1][0][i], KS == 1 || ok);
        WP<WB> wu = cook_wp<WB>(wb[rl & 1][1][i], KS == 1 || ok);
        if constexpr (WB == WB_MX) {
          const int o = (wr * RW + rl) * nblk + lane + 64 * i;
          wg.s = ok ? e8m0_float(msc[o]) : 0.0f;
          wu.s = ok ? e8m0_float(msc[MSC + o]) : 0.0f;
        }
        if constexpr (WB == WB_F8) {
          const int o = (ok ? p0 + lane + 64 * i : p0) >> 3;
          const float *fs = reinterpret_cast<const float *>(msc);
          wg.s = ok ? fs[o] : 0.0f;
          wu.s = ok ? fs[F8_MSC + o] : 0.0f;
        }
        rg[i] = ready<WB>(wg);
        ru[i] = ready<WB>(wu);
      }
      const float sg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), rl));
      const float su = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), RW + rl));
      for (int c0 = 0; c0 < ng; c0 += TT) {
        if constexpr (WB == WB_F8) {
#pragma unroll
          for (int i = 0; i < NPL; i++) {
            fresh_codes<WB>(rg[i].p.w);
            fresh_codes<WB>(ru[i].p.w);
          }
        }
        Act<WB> act[NPL][TT];
#pragma unroll
        for (int t = 0; t < TT; t++) {
          const int tok = c0 + t < ng ? c0 + t : c0;
#pragma unroll
          for (int i = 0; i < NPL; i++) {
            const int p = p0 + lane + 64 * i;  // < KS NPL 64 = P
            uint32_t w[AW::N];
#pragma unroll
            for (int q = 0; q < AW::NQ; q++) {
              const uint4 v = aq[(tok * AW::NQ + q) * P + p];
              w[4 * q] = v.x;
              w[4 * q + 1] = v.y;
              w[4 * q + 2] = v.z;
              w[4 * q + 3] = v.w;
            }
#pragma unroll
            for (int j = 0; j < AW::NS; j++) w[4 * AW::NQ + j] = __float_as_uint(as[(tok * AW::NS + j) * P + p]);
            __builtin_memcpy(&act[i][t], w, sizeof(w));
          }
        }
        float g[TT], u[TT];
#pragma unroll
        for (int t = 0; t < TT; t++) g[t] = u[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; i++) {
#pragma unroll
          for (int t = 0; t < TT; t++) {
            const PDots<WB> dg = ready_idot<WB>(rg[i], act[i][t]);
            g[t] += pdots_value<WB>(dg, act[i][t], ready_scale<WB>(rg[i]));
            const PDots<WB> du = ready_idot<WB>(ru[i], act[i][t]);
            u[t] += pdots_value<WB>(du, act[i][t], ready_scale<WB>(ru[i]));
            if constexpr (DBG) {
              const int p = p0 + lane + 64 * i;
              const bool ok = p < pend && c0 + t < ng;
              const int pr = pairs[g0 + min(c0 + t, ng - 1)];
              if (a.dbg.ffn.gate_dots)
                dump_pdots<WB>(a.dbg.ffn.gate_dots, dg, pr, rbase + rl, I, H / 32, p, ok);
              if (a.dbg.ffn.up_dots)
                dump_pdots<WB>(a.dbg.ffn.up_dots, du, pr, rbase + rl, I, H / 32, p, ok);
            }
          }
        }
#pragma unroll
        for (int t = 0; t < TT; t++) {
          const float gv = sg * wave_sum(g[t]);
          const float uv = su * wave_sum(u[t]);
          if (lane == 0 && c0 + t < ng) {
            if constexpr (KS == 1) {
              hbs[c0 + t][wv * 8 + rl] = silu(gv) * uv;
              if (DBG && a.dbg.ffn.h)
                a.dbg.ffn.h[(size_t)pairs[g0 + c0 + t] * I + blk * 32 + wv * 8 + rl] =
                    silu(gv) * uv;
            } else {
              part[khalf][c0 + t][wr * RW + rl][0] = gv;
              part[khalf][c0 + t][wr * RW + rl][1] = uv;
            }
          }
        }
      }
    }
    if constexpr (KS == 2) {  // the halves added, as gate_up_rows does
      __syncthreads();
      if (tid < ng * 32) {
        const int t = tid >> 5, r = tid & 31;
        hbs[t][r] = silu(part[0][t][r][0] + part[1][t][r][0]) *
                    (part[0][t][r][1] + part[1][t][r][1]);
        if (DBG && a.dbg.ffn.h) a.dbg.ffn.h[(size_t)pairs[g0 + t] * I + blk * 32 + r] = hbs[t][r];
      }
    }
    __syncthreads();
    if (tid < ng * 8) {  // Q8_0 of each token's 32 h values
      const int t = tid >> 3, j = tid & 7;
      int k0, ks, off;
      h_word<WB>(blk, j, k0, ks, off);
      const float4 v = make_float4(hbs[t][k0], hbs[t][k0 + ks], hbs[t][k0 + 2 * ks],
                                   hbs[t][k0 + 3 * ks]);
      float dd;
      const uint32_t packed = q8_quad(v, &dd);
      const int pair = min(max(pairs[g0 + t], 0), a.T * (a.K + a.n_shared) - 1);
      *reinterpret_cast<uint32_t *>(a.qh + (size_t)pair * I + off) = packed;
      if (j == 0) a.dh[(size_t)pair * (I / 32) + blk] = dd;
      if (DBG) dump_q8_word(a.dbg.ffn.q_h, a.dbg.ffn.d_h, pair, I, blk, k0, ks, packed, dd, j == 0);
    }
  }
}

// ============================================================ K1b: selection + shared gate/up

// The shared expert's gate/up (it needs no routing), in workgroups of 4 SRW
// rows so that its bytes spread over every CU: wave wv holds rows
// 4 SRW blk + SRW wv .. (a gate and an up row each) and runs every token
// through them;
// h goes out in fp32 (its Q8_0 blocks span four workgroups; the gate/up
// kernel quantises them).
template <int WB, int TT, int NPL, int SRW, bool DBG>
__device__ void shared_rows_block(const LayerArgs &a, int blk) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I, T = a.T;
  const int npieces = H / (128 / code_bits<WB>());
  const size_t row_b = (size_t)H * code_bits<WB>() / 8;
  const uint8_t *gate = a.shared;
  const uint8_t *up = a.shared + (size_t)I * row_b;
  const uint8_t *tail = a.shared + 3 * (size_t)I * row_b;
  const int nblk = H / 32;
  // the scales the piece loads take for row r of gate (m = 0) or up: MXFP4
  // the row's E8M0 bytes, FP8 its 128-row block's fp32 scales
  auto scl = [&](int m, size_t r) -> const uint8_t * {
    if constexpr (WB == WB_F8)
      return tail + 4 * ((size_t)m * (I / 128) * (H / 128) + (r >> 7) * (H / 128));
    else
      return tail + ((size_t)m * I + r) * nblk;
  };
  const int r0 = blk * 4 * SRW + wv * SRW;
  // Everything unconditional (lanes past the row read its first piece and
  // get zero activations), the first tokens' activations (cache hits) ahead
  // of the weights: one round trip for all.
  auto load_acts = [&](ActRaw<WB> (&dst)[NPL][TT], int c0) {
#pragma unroll
    for (int t = 0; t < TT; t++) {
      const int tok = c0 + t < T ? c0 + t : c0;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        dst[i][t] = load_act_raw<WB>(a.q + (size_t)tok * H, a.d + (size_t)tok * (H / 32),
                                     p < npieces ? p : 0, true);
      }
    }
  };
  ActRaw<WB> araw[NPL][TT];
  load_acts(araw, 0);
  WRaw<WB> wb[SRW][2][NPL];
#pragma unroll
  for (int rr = 0; rr < SRW; rr++) {
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      const int p = lane + 64 * i;
      const int pc = p < npieces ? p : 0;
      const size_t r = (size_t)(r0 + rr);
      wb[rr][0][i] = load_wraw<WB>(gate + r * row_b, scl(0, r), pc);
      wb[rr][1][i] = load_wraw<WB>(up + r * row_b, scl(1, r), pc);
    }
  }
  // no row scales: MXFP4 1, FP8 1/512 (its codes enter as 512 x value)
  constexpr bool blk_scaled = WB == WB_MX || WB == WB_F8;
  constexpr float unit = WB == WB_F8 ? 1.0f / 512.0f : 1.0f;
  float sg[SRW], su[SRW];
#pragma unroll
  for (int rr = 0; rr < SRW; rr++) {
    sg[rr] = blk_scaled ? unit : gload<float>(tail, 4 * (size_t)(r0 + rr));
    su[rr] = blk_scaled ? unit : gload<float>(tail, 4 * ((size_t)I + r0 + rr));
  }
  for (int c0 = 0; c0 < T; c0 += TT) {
#pragma unroll
    for (int rr = 0; rr < SRW; rr++)
#pragma unroll
      for (int m = 0; m < 2; m++)
#pragma unroll
        for (int i = 0; i < NPL; i++) fresh_codes<WB>(wb[rr][m][i].w);
    if (c0 > 0) load_acts(araw, c0);
    Act<WB> act[NPL][TT];
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      const bool ok = lane + 64 * i < npieces;
#pragma unroll
      for (int t = 0; t < TT; t++) act[i][t] = cook_act<WB>(ok ? araw[i][t] : ActRaw<WB>{});
    }
#pragma unroll
    for (int rr = 0; rr < SRW; rr++) {
      float g[TT], u[TT];
#pragma unroll
      for (int t = 0; t < TT; t++) g[t] = u[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const WReady<WB> rg = ready<WB>(cook_wp<WB>(wb[rr][0][i], true));
        const WReady<WB> ru = ready<WB>(cook_wp<WB>(wb[rr][1][i], true));
#pragma unroll
        for (int t = 0; t < TT; t++) {
          const PDots<WB> dg = ready_idot<WB>(rg, act[i][t]);
          g[t] += pdots_value<WB>(dg, act[i][t], ready_scale<WB>(rg));
          const PDots<WB> du = ready_idot<WB>(ru, act[i][t]);
          u[t] += pdots_value<WB>(du, act[i][t], ready_scale<WB>(ru));
          if constexpr (DBG) {  // pair T*K + token of the shared expert
            const int p = lane + 64 * i;
            const bool ok = p < npieces && c0 + t < T;
            const int pr = a.T * a.K + min(c0 + t, T - 1);
            if (a.dbg.ffn.gate_dots)
              dump_pdots<WB>(a.dbg.ffn.gate_dots, dg, pr, r0 + rr, I, H / 32, p, ok);
            if (a.dbg.ffn.up_dots)
              dump_pdots<WB>(a.dbg.ffn.up_dots, du, pr, r0 + rr, I, H / 32, p, ok);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < TT; t++) {
        const float gv = sg[rr] * wave_sum(g[t]);
        const float uv = su[rr] * wave_sum(u[t]);
        if (lane == 0 && c0 + t < T) {
          a.hs[(size_t)(c0 + t) * I + r0 + rr] = silu(gv) * uv;
          if (DBG && a.dbg.ffn.h)
            a.dbg.ffn.h[(size_t)(a.T * a.K + c0 + t) * I + r0 + rr] = silu(gv) * uv;
        }
      }
    }
  }
}

// Workgroups [0, T): selection of token blockIdx.x; the rest: shared rows.
template <int WB, int TT, int NPL, bool DBG>
__global__ void __launch_bounds__(256) k_select_small(LayerArgs a) {
  __shared__ SelLds sm;
  if ((int)blockIdx.x >= a.T) {
    // tokens per chunk of the shared rows (their weights stay in registers,
    // so only the chain of activation round trips grows with T)
    constexpr int STT = TT == 1 ? 1 : (WB == 4 || WB == WB_MX) ? MOE_SHARED_TT : TT;
    shared_rows_block<WB, STT, NPL, shared_rpw(TT), DBG>(a, blockIdx.x - a.T);
    return;
  }
  select_token(a, sm, blockIdx.x);
}

// ============================================================ K2: gate/up

// Expert slot j of the batch union (the j-th smallest distinct expert in
// idx) and its pairs in slot order, built in LDS by every K2 workgroup from
// the T*K selections: bitmap of chosen experts, an expert's slot = chosen
// experts below it, pairs ranked by ballots.  ent: expert (-1 = none), count,
// TMAX pair ids, TMAX token ids.  Returns the expert's record address; with a
// table of record pointers, every thread holding a selection fetches its
// entry at once, so that load overlaps the union's own work.
__device__ const uint8_t *union_slot(const LayerArgs &a, int j, int *ent) {
  __shared__ uint32_t bits[32];
  __shared__ int wcnt[4];
  __shared__ const uint8_t *rec;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = a.T * a.K, E = a.E;
  if (tid < 32) bits[tid] = 0u;
  if (tid == 0) {
    ent[0] = -1;
    rec = a.shared;  // any readable address for an empty slot
  }
  int e = -1;  // -1: no pair, or a rank dropped by top-p
  if (tid < n) {
    const int v = a.idx[tid];
    e = (v >= 0 && v < E) ? v : -1;
  }
  const uint8_t *my_rec = e >= 0 ? expert_record(a, e) : nullptr;
  __syncthreads();
  if (e >= 0) atomicOr(&bits[e >> 5], 1u << (e & 31));
  __syncthreads();
  if (e >= 0) {
    int r = __popc(bits[e >> 5] & ((1u << (e & 31)) - 1u));
    for (int w = 0; w < (e >> 5); w++) r += __popc(bits[w]);
    if (r == j) {  // every holder of that expert writes the same values
      ent[0] = e;
      rec = my_rec;
    }
  }
  __syncthreads();
  const int ej = ent[0];
  const bool m = tid < n && e == ej && ej >= 0;
  const unsigned long long b = __ballot(m);
  if (lane == 0) wcnt[wv] = __popcll(b);
  __syncthreads();
  int rank = __popcll(b & ((1ull << lane) - 1ull));
  for (int w = 0; w < wv; w++) rank += wcnt[w];
  if (m && rank < sbk::TMAX) {  // a token picks an expert at most once
    ent[2 + rank] = tid;
    ent[2 + sbk::TMAX + rank] = tid / a.K;
  }
  if (tid == 0) ent[1] = ej >= 0 ? wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3] : 0;
  __syncthreads();
  return rec;
}

// Debug dump (moe_layer_debug) of the batch union in moe_group's format,
// written by the row-block-0 workgroup of each slot j from its entry ent
// (expert ej, count, pair ids): counts and offsets of the experts
// (previous selected expert, ej], active[j], ej's part of perm and inv; slot
// 0 also marks the dropped ranks (inv -1), and the last selected expert's
// slot fills what follows it (counts, offsets, active, the perm tail,
// n_active).
__device__ void union_dump(const LayerArgs &a, int j, const int *ent) {
  __shared__ int s_off, s_tot, s_prev, s_next;
  const int tid = threadIdx.x, n = a.T * a.K, E = a.E;
  const int ej = ent[0], cnt = ent[1];
  const moe_layer_debug &g = a.dbg;
  if (tid == 0) {
    s_off = 0;
    s_tot = 0;
    s_prev = -1;
    s_next = E;
  }
  __syncthreads();
  int e = -1;
  if (tid < n) {
    const int v = a.idx[tid];
    e = (v >= 0 && v < E) ? v : -1;
  }
  if (e >= 0) {
    atomicAdd(&s_tot, 1);
    if (e < ej) {
      atomicAdd(&s_off, 1);
      atomicMax(&s_prev, e);
    }
    if (e > ej) atomicMin(&s_next, e);
  }
  __syncthreads();
  if (j == 0 && tid < n && e < 0) g.inv[tid] = -1;
  if (ej < 0) return;  // past the union
  const int off = s_off, tot = s_tot;
  for (int x = s_prev + 1 + tid; x <= ej; x += 256) {
    g.counts[x] = x == ej ? cnt : 0;
    g.offsets[x] = off;
  }
  if (tid < cnt) {
    g.perm[off + tid] = ent[2 + tid];
    g.inv[ent[2 + tid]] = off + tid;
  }
  if (tid == 0) g.active[j] = ej;
  if (s_next == E) {  // the largest selected expert
    for (int x = ej + 1 + tid; x <= E; x += 256) {
      if (x < E) g.counts[x] = 0;
      g.offsets[x] = tot;
    }
    for (int m = j + 1 + tid; m < E; m += 256) g.active[m] = -1;
    for (int i = tot + tid; i < n; i += 256) g.perm[i] = -1;
    if (tid == 0) *g.n_active = j + 1;
  }
}

// Block (blk, j): rows 32 blk .. 32 blk + 31 of h for routed slot j.  The
// workgroups with blk == 0 also publish their slot's table entry (and the
// shared expert's) for the down kernel.
template <int WB, int TT, int NPL, bool DBG>
__global__ void __launch_bounds__(256, WB == WB_MX && TT > 1 ? 2 : 1) k_gate_up_small(LayerArgs a) {
  __shared__ float hb[TT][32];
  __shared__ int ent[SLOT_W];
  __shared__ __align__(16) uint8_t msc[gu_msc_bytes<WB>()];
  const int j = blockIdx.y, blk = blockIdx.x;
  if (j == 0 && a.n_shared && (int)threadIdx.x < a.T * 8) {
    // Q8_0 of the shared expert's h, block blk of every token
    const int t = threadIdx.x >> 3, q = threadIdx.x & 7;
    int k0, ks, off;
    h_word<WB>(blk, q, k0, ks, off);
    const float *hrow = a.hs + (size_t)t * a.I + blk * 32;
    const float4 v = make_float4(hrow[k0], hrow[k0 + ks], hrow[k0 + 2 * ks], hrow[k0 + 3 * ks]);
    float dd;
    const uint32_t packed = q8_quad(v, &dd);
    const int pair = a.T * a.K + t;
    *reinterpret_cast<uint32_t *>(a.qh + (size_t)pair * a.I + off) = packed;
    if (q == 0) a.dh[(size_t)pair * (a.I / 32) + blk] = dd;
    if (DBG) dump_q8_word(a.dbg.ffn.q_h, a.dbg.ffn.d_h, pair, a.I, blk, k0, ks, packed, dd, q == 0);
  }
  const uint8_t *rec = union_slot(a, j, ent);
  if (DBG && blk == 0 && a.dbg.counts) union_dump(a, j, ent);
  const int n_tok = min(max(ent[1], 0), a.T);
  if (blk == 0) {
    int32_t *dst = a.slots + (size_t)(a.n_shared + j) * SLOT_W;
    if (threadIdx.x < SLOT_PTR) dst[threadIdx.x] = ent[threadIdx.x];
    if (threadIdx.x == 0) *reinterpret_cast<const uint8_t **>(dst + SLOT_PTR) = rec;
    if (j == 0 && a.n_shared && threadIdx.x < a.T) {  // the shared expert takes every token
      if (threadIdx.x == 0) {
        a.slots[0] = -1;
        a.slots[1] = a.T;
        *reinterpret_cast<const uint8_t **>(a.slots + SLOT_PTR) = a.shared;
      }
      a.slots[2 + threadIdx.x] = a.T * a.K + threadIdx.x;
      a.slots[2 + sbk::TMAX + threadIdx.x] = threadIdx.x;
    }
  }
  if (n_tok == 0) return;
  const int *pairs = ent + 2, *toks = ent + 2 + sbk::TMAX;
  // int8 rows longer than 4 pieces per lane are split over two waves
  constexpr int KS = byte_codes(WB) && NPL > 4 ? 2 : 1;
  auto qrow = [&](int i) {
    return (const int8_t *)(a.q + (size_t)min(max(toks[i], 0), a.T - 1) * a.H);
  };
  auto drow = [&](int i) {
    return (const float *)(a.d + (size_t)min(max(toks[i], 0), a.T - 1) * (a.H / 32));
  };
  constexpr int NPLK = KS == 2 ? (NPL + 1) / 2 : NPL;  // pieces per lane of a wave's share of a row
  if constexpr (TT > 1 && MOE_GU_LDS) {
    if constexpr (gu_stage_tokens<WB, TT, NPLK, KS>() >= 2 * TT) {
      if (n_tok > TT) {  // several chunks: rows streamed once for all of them
        gate_up_rows_lds<WB, TT, NPLK, KS, DBG>(a, msc, rec, blk, n_tok, pairs, qrow, drow);
        return;
      }
    }
  }
  gate_up_rows<WB, TT, NPLK,
               (TT == 1 ? (WB == 2 ? 2 * MOE_K2_ROWS : byte_codes(WB) || WB == WB_MX ? 1 : MOE_K2_ROWS) : 1),
               KS, DBG>(
      a, hb, msc, rec, blk, n_tok, pairs, qrow, drow);
}

// ============================================================ K3: down + combine

// Sum over each row of 16 lanes (every lane of the row gets it).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x128>(v);  // row_ror:8
  return v;
}

// Sum over each group of 8 lanes (quads, then the half-row mirror).
__device__ __forceinline__ float row8_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror: lane i + lane 7-i of each 8
  return v;
}

template <int LPR>
__device__ __forceinline__ float lane_row_sum(float v) {
  return LPR == 16 ? row16_sum(v) : row8_sum(v);
}

constexpr int TAB_W = 2 + sbk::TMAX;  // expert, count, pairs: what the down kernel reads

// Activations of pairs prs[c0 .. c0+TT) (pair ids clamped, -1 past n_tok)
// for the pieces qb + pl + LPR i of a quarter of nq pieces.
template <int WB, int TT, int NPQ, int LPR>
__device__ __forceinline__ void down_act(const LayerArgs &a, const int *prs, int n_tok, int c0,
                                         int P, int qb, int nq, int pl,
                                         ActRaw<WB> (&act)[NPQ][TT],
                                         int (&pair)[TT]) {
  const int I = a.I;
#pragma unroll
  for (int t = 0; t < TT; t++) {
    pair[t] = (c0 + t < n_tok) ? min(max(prs[c0 + t], 0), P - 1) : -1;
    const int pp = pair[t] >= 0 ? pair[t] : 0;
#pragma unroll
    for (int i = 0; i < NPQ; i++) {
      const int q = pl + LPR * i;
      // always a valid piece (piece 0 of the row, pair 0 for a missing
      // pair), so that no branch holds the load: lanes past the quarter
      // have zero weights, and missing pairs are never stored
      const bool ok = pair[t] >= 0 && q < nq;
      act[i][t] = load_act_raw<WB>(a.qh + (size_t)pp * I, a.dh + (size_t)pp * (I / 32),
                                   ok ? qb + q : 0, true);
    }
  }
}

// Where the down kernel's debug dumps go: block dots [pair][H][I/32] of the
// rows j0 + ..., pieces qb + ... of the row (null: no dump).
struct DownDump {
  int32_t *dots;
  int H, nblk, j0, qb;
};

// The RPL = LPR/8 rows of lane row rl (rl, rl + 64/LPR) of one slot for TT
// pairs: quarter partials into part[wv][pair][row].
template <int WB, int TT, int NPQ, int LPR, bool DBG>
__device__ __forceinline__ void down_rows(float *part, int P, int wv, int rl, int pl, int nq,
                                          const WRaw<WB> (&w)[LPR / 8][NPQ],
                                          const float (&sd)[LPR / 8],
                                          const ActRaw<WB> (&raw)[NPQ][TT],
                                          const int (&pair)[TT], const DownDump &dd) {
  Act<WB> act[NPQ][TT];  // rearranged here, where the loads are first needed
#pragma unroll
  for (int i = 0; i < NPQ; i++)
#pragma unroll
    for (int t = 0; t < TT; t++) act[i][t] = cook_act_h<WB>(raw[i][t]);
#pragma unroll
  for (int rr = 0; rr < LPR / 8; rr++) {
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < NPQ; i++) {
      const WReady<WB> rw = ready<WB>(cook_wp<WB>(w[rr][i], pl + LPR * i < nq));
#pragma unroll
      for (int t = 0; t < TT; t++) {
        const PDots<WB> dt = ready_idot<WB>(rw, act[i][t]);
        acc[t] += pdots_value<WB>(dt, act[i][t], ready_scale<WB>(rw));
        if constexpr (DBG) {
          if (dd.dots)
            dump_pdots<WB>(dd.dots, dt, max(pair[t], 0), dd.j0 + rl + (64 / LPR) * rr, dd.H,
                           dd.nblk, dd.qb + pl + LPR * i, pair[t] >= 0 && pl + LPR * i < nq);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TT; t++) {
      const float yv = sd[rr] * lane_row_sum<LPR>(acc[t]);
      if (pl == 0 && pair[t] >= 0)
        part[((size_t)wv * P + pair[t]) * sbk::RT + rl + (64 / LPR) * rr] = yv;
    }
  }
}

// Block `tile`: output rows 8 tile .. 8 tile + 7 of every expert slot for
// every token.  Wave wv covers all 8 rows over quarter wv of the I
// dimension (pieces [wv n/4, (wv+1) n/4) of the row's n) with LPR lanes per
// row: lane l takes rows l/LPR (+ 64/LPR) and the pieces l%LPR (+LPR i) of
// the quarter, so the lane rows of a wave share each activation piece (one
// cache-line request for all).  LPR = 8 when a quarter has at most 8 pieces,
// so that every lane loads.  Rows are reduced over their LPR lanes; the 4
// quarters land in LDS and are added in quarter order in the combine, which
// runs in rank order:
//   y[t] = residual[t] + shared[t] + sum_k w[t,k] * expert_k[t]
template <int WB, int TT, int NPQ, int SB, int LPR, bool PIPE, bool SH, bool DBG>
__global__ void __launch_bounds__(256) k_down_small(LayerArgs a) {
  constexpr int RPL = LPR / 8;  // rows per lane
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ float wsh[256];
  const int tile = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const int P = T * (K + a.n_shared);  // pairs
  float *part = reinterpret_cast<float *>(dyn);                          // [4][P][RT]
  int *tab = reinterpret_cast<int *>(dyn + (size_t)4 * P * sbk::RT * 4);  // [slots][TAB_W]
  const uint8_t **recs = reinterpret_cast<const uint8_t **>(
      dyn + (size_t)4 * P * sbk::RT * 4 + (((size_t)a.n_slots_ub * TAB_W * 4 + 7) & ~(size_t)7));
  constexpr int CB = code_bits<WB>();
  const int npieces = I / (128 / CB);
  const int qb = wv * npieces / 4, nq = (wv + 1) * npieces / 4 - qb;  // this wave's quarter
  const size_t row_b = (size_t)I * CB / 8;
  const size_t down_off = 2 * (size_t)I * ((size_t)H * CB / 8);
  const size_t tail_off = 3 * (size_t)I * ((size_t)H * CB / 8);  // scales after the codes
  const size_t dsc_off = tail_off + 2 * (size_t)I * (H / 32);    // MXFP4 down block scales
  const int nblk = I / 32;
  // the scales the piece loads take for down row `row` of a record: MXFP4
  // the row's E8M0 bytes, FP8 its 128-row block's fp32 scales; the row
  // scale (MXFP4 none, FP8 1/512: its codes enter as 512 x value)
  auto dscl = [&](const uint8_t *blob, int row) -> const uint8_t * {
    if constexpr (WB == WB_F8)
      return blob + tail_off +
             4 * ((size_t)2 * (I / 128) * (H / 128) + (size_t)(row >> 7) * (I / 128));
    else
      return blob + dsc_off + (size_t)row * nblk;
  };
  auto drow_scale = [&](const uint8_t *blob, int row) -> float {
    if constexpr (WB == WB_MX) return 1.0f;
    else if constexpr (WB == WB_F8) return 1.0f / 512.0f;
    else return gload<float>(blob, tail_off + 4 * ((size_t)2 * I + row));
  };
  const int rl = lane / LPR, pl = lane % LPR;
  const int j0 = tile * sbk::RT;
  const DownDump ddump{DBG ? a.dbg.ffn.down_dots : nullptr, H, I / 32, j0, qb};
  // The slot table (its first 256 entries, one per thread), the combine
  // weights and the residual are requested first, then the shared expert's
  // rows and first TT pairs (they need nothing from the table): the table
  // arrives after one plain round trip, and the routed rows are requested
  // while the shared ones are still in flight.  Every load is unconditional
  // (clamped indices; the residual falls back to x, same shape), so that
  // storing the table waits for the table alone.
  const int ntab = a.n_slots_ub * TAB_W;
  const int tab_i = min(tid, ntab - 1);
  const int tab_v = a.slots[(size_t)(tab_i / TAB_W) * SLOT_W + tab_i % TAB_W];
  const int rec_i = min(tid, a.n_slots_ub - 1);
  const uint8_t *rec_v =
      *reinterpret_cast<const uint8_t *const *>(a.slots + (size_t)rec_i * SLOT_W + SLOT_PTR);
  const float w_v = a.w[min(tid, T * K - 1)];
  const int v = tid;  // combine: one thread per (token, row), T * RT <= 128
  const bool comb = v < T * sbk::RT;
  const int vc = min(v, T * sbk::RT - 1);
  const float *res_p = a.residual ? a.residual : a.x;
  const float res_v = res_p[(size_t)(vc / sbk::RT) * H + j0 + vc % sbk::RT];
  int shp[sbk::TMAX];  // the shared expert's pair ids T*K + t
#pragma unroll
  for (int t = 0; t < sbk::TMAX; t++) shp[t] = T * K + t;
  constexpr int S0 = SH ? 1 : 0;
  WRaw<WB> ws0[RPL][NPQ];
  float sd0[RPL];
  ActRaw<WB> act_s[NPQ][TT];
  int pair_s[TT];
  if constexpr (SH) {
    const uint8_t *down = a.shared + down_off;
#pragma unroll
    for (int rr = 0; rr < RPL; rr++) {
      const int row = j0 + rl + (64 / LPR) * rr;
#pragma unroll
      for (int i = 0; i < NPQ; i++) {
        const int q = pl + LPR * i;
        ws0[rr][i] = load_wraw<WB>(down + (size_t)row * row_b, dscl(a.shared, row),
                                   q < nq ? qb + q : qb);
      }
      sd0[rr] = drow_scale(a.shared, row);
    }
    down_act<WB, TT, NPQ, LPR>(a, shp, T, 0, P, qb, nq, pl, act_s, pair_s);
  }
  // (threads past the end store their clamped entry again, the same value:
  // a store behind a branch would draw its load into the branch)
  tab[tab_i] = tab_v;
  for (int i = tid + 256; i < ntab; i += 256)  // batches of many tokens
    tab[i] = a.slots[(size_t)(i / TAB_W) * SLOT_W + i % TAB_W];
  recs[rec_i] = rec_v;
  for (int i = tid + 256; i < a.n_slots_ub; i += 256)
    recs[i] = *reinterpret_cast<const uint8_t *const *>(a.slots + (size_t)i * SLOT_W + SLOT_PTR);
  wsh[min(tid, T * K - 1)] = w_v;
  const float resid = (comb && a.residual) ? res_v : 0.0f;
  __syncthreads();
  int n_slots = 0;
  while (n_slots < a.n_slots_ub && tab[n_slots * TAB_W + 1] > 0) n_slots++;

  // Routed slots SB at a time, double-buffered: the rows and first pairs of
  // the next SB slots are in flight while these are reduced.  A slot past
  // the last (the prefetch after the final batch) reads the last slot's
  // rows again, which the cache still holds, and nothing of it is stored:
  // every load is unconditional.
  struct Batch {
    WRaw<WB> wd[SB][RPL][NPQ];
    float sd[SB][RPL];
    ActRaw<WB> act0[SB][NPQ][TT];
    int pair0[SB][TT];
  };
  auto load_batch = [&](Batch &bt, int s0) {
#pragma unroll
    for (int b = 0; b < SB; b++) {
      const int sl = min(s0 + b, n_slots - 1);  // n_slots >= 1: every token has a routed expert
      const uint8_t *blob = recs[sl];
      const uint8_t *down = blob + down_off;
#pragma unroll
      for (int rr = 0; rr < RPL; rr++) {
        const int row = j0 + rl + (64 / LPR) * rr;
#pragma unroll
        for (int i = 0; i < NPQ; i++) {
          const int q = pl + LPR * i;
          bt.wd[b][rr][i] = load_wraw<WB>(down + (size_t)row * row_b, dscl(blob, row),
                                          q < nq ? qb + q : qb);
        }
        bt.sd[b][rr] = drow_scale(blob, row);
      }
      const int n_tok = s0 + b < n_slots ? min(tab[sl * TAB_W + 1], T) : 0;
      down_act<WB, TT, NPQ, LPR>(a, tab + sl * TAB_W + 2, n_tok, 0, P, qb, nq, pl, bt.act0[b],
                                 bt.pair0[b]);
    }
  };
  auto run_batch = [&](const Batch &bt, int s0) {
#pragma unroll
    for (int b = 0; b < SB; b++) {
      const int sl = min(s0 + b, a.n_slots_ub - 1);
      const int n_tok = s0 + b < n_slots ? min(tab[sl * TAB_W + 1], T) : 0;
      down_rows<WB, TT, NPQ, LPR, DBG>(part, P, wv, rl, pl, nq, bt.wd[b], bt.sd[b], bt.act0[b],
                                  bt.pair0[b], ddump);
      for (int c0 = TT; c0 < n_tok; c0 += TT) {
        ActRaw<WB> act[NPQ][TT];
        int pair[TT];
        down_act<WB, TT, NPQ, LPR>(a, tab + sl * TAB_W + 2, n_tok, c0, P, qb, nq, pl, act, pair);
        down_rows<WB, TT, NPQ, LPR, DBG>(part, P, wv, rl, pl, nq, bt.wd[b], bt.sd[b], act, pair,
                                         ddump);
      }
    }
  };
  Batch ba, bb;
  if constexpr (PIPE) load_batch(ba, S0);  // requested before the shared slot is reduced
  if (S0) {  // the shared slot, from the registers filled above
    down_rows<WB, TT, NPQ, LPR, DBG>(part, P, wv, rl, pl, nq, ws0, sd0, act_s, pair_s, ddump);
    for (int c0 = TT; c0 < T; c0 += TT) {
      ActRaw<WB> act[NPQ][TT];
      int pair[TT];
      down_act<WB, TT, NPQ, LPR>(a, shp, T, c0, P, qb, nq, pl, act, pair);
      down_rows<WB, TT, NPQ, LPR, DBG>(part, P, wv, rl, pl, nq, ws0, sd0, act, pair, ddump);
    }
  }
  if constexpr (PIPE) {
    for (int s0 = S0; s0 < n_slots; s0 += 2 * SB) {
      load_batch(bb, s0 + SB);
      run_batch(ba, s0);
      if (s0 + SB >= n_slots) break;
      load_batch(ba, s0 + 2 * SB);
      run_batch(bb, s0 + SB);
    }
  } else {  // one batch at a time (fewer registers)
    for (int s0 = S0; s0 < n_slots; s0 += SB) {
      load_batch(ba, s0);
      run_batch(ba, s0);
    }
  }
  __syncthreads();
  // combine in rank order, one thread per (token, row); quarters in order
  const bool norm = a.y_norm != nullptr;
  float ss = 0.0f;
  if (comb) {
    const int t = v / sbk::RT, r = v % sbk::RT, j = j0 + r;
    auto full = [&](int pr) {
      const size_t q = (size_t)P * sbk::RT;
      const float *pp = part + (size_t)pr * sbk::RT + r;
      return ((pp[0] + pp[q]) + pp[2 * q]) + pp[3 * q];
    };
    float acc = resid;
    if (a.n_shared) acc += full(T * K + t);
    for (int k = 0; k < K; k++) {
      const float wk = wsh[t * K + k];
      if (wk != 0.0f) acc = fmaf(wk, full(t * K + k), acc);  // 0: dropped by top-p
    }
    a.y[(size_t)t * H + j] = acc;
    ss = acc * acc;
  }
  if (!norm) return;
  // per-token sum of squares of this tile's 8 rows (8 consecutive threads);
  // the normalisation kernel adds the tiles
  ss += __shfl_xor(ss, 1, 8);
  ss += __shfl_xor(ss, 2, 8);
  ss += __shfl_xor(ss, 4, 8);
  if (comb && (v % sbk::RT) == 0) a.ssq[(size_t)(v / sbk::RT) * gridDim.x + tile] = ss;
}

// y[t] = residual[t] + shared[t] + sum_k w[t,k] expert_k[t] in rank order
// (w = 0: dropped by top-p, skipped) from the MFMA down's per-pair rows, one
// thread per (t, j) over T x H/256 workgroups; with y_norm, the per-8-row
// sums of squares for k_norm_small as the down kernel above writes them.
__global__ void __launch_bounds__(256) k_combine_small(LayerArgs a) {
  const int t = blockIdx.x, j = blockIdx.y * 256 + threadIdx.x;
  const int H = a.H, K = a.K;
  float acc = 0.0f, ss = 0.0f;
  if (j < H) {
    acc = a.residual ? a.residual[(size_t)t * H + j] : 0.0f;
    if (a.n_shared) acc += a.eo_s[(size_t)t * H + j];
    for (int k = 0; k < K; k++) {
      const float wk = a.w[t * K + k];
      if (wk != 0.0f) acc = fmaf(wk, a.eo_r[((size_t)t * K + k) * H + j], acc);
    }
    a.y[(size_t)t * H + j] = acc;
    ss = acc * acc;
  }
  if (!a.y_norm) return;
  ss += __shfl_xor(ss, 1, 8);
  ss += __shfl_xor(ss, 2, 8);
  ss += __shfl_xor(ss, 4, 8);
  if (j < H && (j % sbk::RT) == 0) a.ssq[(size_t)t * (H / sbk::RT) + j / sbk::RT] = ss;
}

// ============================================================ K4: RMSNorm

// y_norm[t] = y[t] / sqrt(sum(y[t]^2) / H + eps) for the next layer of a
// pre-norm stack (unit gain).  Workgroup (t, c): every workgroup of token t
// adds the n_tiles partial sums in the same fixed order (strided per thread,
// then the DPP wave sum, then the 4 waves in order) and scales 1024 values.
__global__ void __launch_bounds__(256) k_norm_small(LayerArgs a, int n_tiles) {
  __shared__ float wsum[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  float p = 0.0f;
  for (int i = tid; i < n_tiles; i += 256) p += a.ssq[(size_t)t * n_tiles + i];
  p = wave_sum(p);
  if ((tid & 63) == 0) wsum[tid >> 6] = p;
  __syncthreads();
  const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float inv = 1.0f / sqrtf(tot / (float)a.H + a.eps);
  const int j = blockIdx.y * 1024 + tid * 4;
  if (j < a.H) {
    float4 y4 = *reinterpret_cast<const float4 *>(a.y + (size_t)t * a.H + j);
    y4.x *= inv;
    y4.y *= inv;
    y4.z *= inv;
    y4.w *= inv;
    *reinterpret_cast<float4 *>(a.y_norm + (size_t)t * a.H + j) = y4;
  }
}

// ============================================================ launch

template <int WB, int TT, int NPG, int NPD, bool DBG>
void launch3(const LayerArgs &a, hipStream_t st, const moe_events *ev) {
  const int n_sh = a.n_shared ? a.I / (4 * shared_rpw(TT)) : 0;
  if (a.T >= MOE_ROUTE_EB2_T && a.E % 2 == 0)
    launch_k(k_route_small<2>, dim3(a.E / 2, 2), dim3(256), 0, st,
             stage_ev(ev, MOE_STAGE_ROUTER_SCORES), a);
  else
    launch_k(k_route_small<1>, dim3(a.E, 1), dim3(256), 0, st,
             stage_ev(ev, MOE_STAGE_ROUTER_SCORES), a);
  launch_k(k_select_small<WB, TT, NPG, DBG>, dim3(a.T + n_sh), dim3(256), 0, st,
           stage_ev(ev, MOE_STAGE_ROUTER_SELECT), a);
  launch_k(k_gate_up_small<WB, TT, NPG, DBG>, dim3(a.I / 32, a.n_slots_ub - a.n_shared), dim3(256), 0,
           st, stage_ev(ev, MOE_STAGE_GATE_UP), a);
  const int P = a.T * (a.K + a.n_shared);
  const size_t lds3 = (size_t)4 * P * sbk::RT * sizeof(float) +
                      (((size_t)a.n_slots_ub * TAB_W * 4 + 7) & ~(size_t)7) +
                      (size_t)a.n_slots_ub * sizeof(void *);
  constexpr int fbit = WB == 4 ? 1 : WB == 2 ? 2 : byte_codes(WB) ? 4 : 8;
  constexpr bool PIPE = (MOE_K3_PIPE & fbit) != 0;
  constexpr int SB = !PIPE ? MOE_K3_SLOTS_NOPIPE
                    : TT == 1 && WB == 2 ? MOE_K3_SLOTS_INT2
                                         : MOE_K3_SLOTS;
  constexpr int TT3 = TT == 1 ? 1 : MOE_K3_TT;  // tokens per chunk in the down kernel
  const int quarter = (a.I / (128 / code_bits<WB>()) + 3) / 4;
  const int mfma_min_t = WB == 4 || WB == 2 ? MOE_DOWN_MFMA_MIN_T
                         : WB == WB_MX        ? MOE_DOWN_MFMA_MIN_T_MX
                                              : MOE_DOWN_MFMA_MIN_T_WIDE;
  if (WB != WB_F8 && a.T >= mfma_min_t && a.H % 64 == 0 && a.I % 64 == 0) {
    // many tokens per expert: the down projection as MFMA tiles of 64 rows
    // x the slot's tokens (activations staged once per 64 rows, not once
    // per 8), then the rank-order combine
    FfnArgs f;
    f.H = a.H;
    f.I = a.I;
    f.E = a.E;
    f.K = a.K;
    f.T = a.T;
    f.n_shared = a.n_shared;
    f.wbits = a.wbits;
    f.wfmt = a.wfmt;
    f.blob_bytes = a.blob_bytes;
    f.q = nullptr;
    f.d = nullptr;
    f.experts = a.experts;
    f.expert_ptrs = a.expert_ptrs;
    f.shared = a.shared;
    f.offsets = f.perm = f.active = f.n_active = nullptr;
    f.h = nullptr;
    f.expert_out = a.eo_r;
    f.shared_out = a.eo_s;
    f.dbg = a.dbg.ffn;
    launch_down_mfma_slots(f, a.slots, a.n_slots_ub, SLOT_W, SLOT_PTR, a.qh, a.dh, DBG, st, ev);
    launch_k(k_combine_small, dim3(a.T, (a.H + 255) / 256), dim3(256), 0, st,
             stage_ev(ev, MOE_STAGE_COMBINE), a);
  } else {
    // with or without a shared expert (its rows are requested unconditionally)
    auto kd = quarter <= 8 ? (a.n_shared ? k_down_small<WB, TT3, 1, SB, 8, PIPE, true, DBG>
                                         : k_down_small<WB, TT3, 1, SB, 8, PIPE, false, DBG>)
                           : (a.n_shared ? k_down_small<WB, TT3, NPD, SB, 16, PIPE, true, DBG>
                                         : k_down_small<WB, TT3, NPD, SB, 16, PIPE, false, DBG>);
    launch_k(kd, dim3(a.H / sbk::RT), dim3(256), (uint32_t)lds3, st,
             stage_ev(ev, MOE_STAGE_DOWN), a);
  }
  if (a.y_norm)
    launch_k(k_norm_small, dim3(a.T, (a.H + 1023) / 1024), dim3(256), 0, st,
             stage_ev(ev, MOE_STAGE_NORM), a, a.H / sbk::RT);
}

template <int WB, int TT, bool DBG>
void launch3_np(const LayerArgs &a, hipStream_t st, const moe_events *ev) {
  const int per = 128 / code_bits<WB>();
  const int ng = (a.H / per + 63) / 64, nd = (a.I / per + 63) / 64;
  if constexpr (byte_codes(WB)) {  // 16 codes per piece: up to 7 pieces per lane
    if (ng <= 2 && nd <= 1) launch3<WB, TT, 2, 1, DBG>(a, st, ev);
    else if (ng <= 4 && nd <= 2) launch3<WB, TT, 4, 2, DBG>(a, st, ev);
    else if (ng <= 6 && nd <= 2) launch3<WB, TT, 6, 2, DBG>(a, st, ev);  // H = 6144: 3 per half
    else launch3<WB, TT, 7, 2, DBG>(a, st, ev);
  } else {
    if (ng <= 1 && nd <= 1) launch3<WB, TT, 1, 1, DBG>(a, st, ev);
    else if (ng <= 2 && nd <= 1) launch3<WB, TT, 2, 1, DBG>(a, st, ev);
    else if (ng <= 3 && nd <= 1) launch3<WB, TT, 3, 1, DBG>(a, st, ev);
    else if (ng <= 4 && nd <= 1) launch3<WB, TT, 4, 1, DBG>(a, st, ev);
    else launch3<WB, TT, 4, 2, DBG>(a, st, ev);
  }
}

// The small-batch step; DBG: the kernels that also write the intermediates
// of a.dbg (moe_layer_debug).
template <bool DBG>
void launch_small_batch_t(LayerArgs a, hipStream_t st, const moe_events *ev) {
  a.n_slots_ub = a.n_shared + (a.T * a.K < a.E ? a.T * a.K : a.E);
  if (a.wfmt == 1) {  // MXFP4: int4 layout of the codes, a scale per piece
    if (a.T == 1) launch3_np<WB_MX, 1, DBG>(a, st, ev);
    else launch3_np<WB_MX, MOE_TT_MX, DBG>(a, st, ev);
  } else if (a.wfmt == 2) {
    // FP8 (1..4 tokens): pieces as int8, one token per chunk (a slot's
    // further tokens are staged in LDS, rows still streamed once): two
    // tokens' converted codes do not fit the registers of the long rows
    launch3_np<WB_F8, 1, DBG>(a, st, ev);
  } else if (a.wbits == 8) {  // a piece carries 16 codes: two tokens per chunk
    if (a.T == 1) launch3_np<8, 1, DBG>(a, st, ev);
    else launch3_np<8, 2, DBG>(a, st, ev);
  } else if (a.wbits == 4) {
    if (a.T == 1) launch3_np<4, 1, DBG>(a, st, ev);
    else launch3_np<4, MOE_TT_INT4, DBG>(a, st, ev);
  } else {
    // an int2 activation fragment covers 64 codes: two tokens per chunk keep
    // the registers within two waves per SIMD
    if (a.T == 1) launch3_np<2, 1, DBG>(a, st, ev);
    else launch3_np<2, 2, DBG>(a, st, ev);
  }
}

}  // namespace
}  // namespace moe

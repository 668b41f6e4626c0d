// Expert FFN for decode and small batches: HBM-streaming GEMV.
//
// Method ("Show HN: 遅いコンピュータで GLM 5.2 を実行する", section
// 実装済みの主な機能: integer-dot, quantisation-kernel and batch-union items):
// packed int4 (or int2) weight codes with one fp32 scale per row are expanded
// on use and multiplied against Q8_0 int8 activations with exact integer
// accumulation per 32-element block; each distinct expert is streamed once
// for all tokens routed to it.
//
// MI355X mapping:
//  * one wave streams whole weight rows: a row of H int4 codes is H/2 bytes,
//    read as 16-byte pieces, lane l taking pieces l, l+64, ...; a wave-wide
//    load is 1 KiB of consecutive bytes (fully coalesced); several rows are
//    loaded before any is consumed so each lane keeps 8-12 loads in flight;
//  * a 16-byte int4 piece is exactly one Q8_0 block (32 codes): nibbles are
//    widened to int8 with two mask/shift ops per word (16 x code), and
//    v_dot4_i32_i8 against the block's even / odd activation bytes gives
//    16 x the exact block dot; the activation bytes are pre-split once per
//    token and reused across all rows;
//  * the fp32 epilogue per block is one int->float conversion and one fma;
//    the wave reduction per row is a 6-step butterfly;
//  * gate and up rows of the same index are processed by the same wave so
//    SwiGLU is fused; h goes to the workspace in fp32 and the down kernel
//    re-quantises it (Q8_0) into LDS in its prologue.
// Grid: x = row tiles, y = expert slot (shared expert first, then the active
// routed experts; slots past n_active exit at once, so no host read-back is
// needed to size the grid).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int GU_RPW = 2;  // gate/up rows per wave (each row: a gate and an up row)
constexpr int DN_RPW = 8;  // down rows per wave

struct SlotInfo {
  const uint8_t *blob;
  int n_tok;
  bool shared;
  const int32_t *list;  // slot ids (routed) or nullptr (shared: tokens 0..T-1)
};

__device__ __forceinline__ bool slot_info(const FfnArgs &a, int j, SlotInfo &si) {
  if (j < a.n_shared) {
    si.blob = a.shared;
    si.n_tok = a.T;
    si.shared = true;
    si.list = nullptr;
    return true;
  }
  const int act = j - a.n_shared;
  if (act >= *a.n_active) return false;
  const int e = a.active[act];
  const int lo = a.offsets[e], hi = a.offsets[e + 1];
  si.blob = expert_record(a, e);
  si.n_tok = hi - lo;
  si.shared = false;
  si.list = a.perm + lo;
  return true;
}

// token index and pair index of the i-th token of a slot
__device__ __forceinline__ void token_of(const FfnArgs &a, const SlotInfo &si, int i, int &tok,
                                         int &pair) {
  if (si.shared) {
    tok = i;
    pair = a.T * a.K + i;
  } else {
    const int s = si.list[i];
    tok = s / a.K;
    pair = s;
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Q8_0 of h for the TT pairs of a down chunk (pair -1: zeros) into LDS:
// codes lq [TT][I], scales ld [TT][I/32]; 8 threads per block of 32, 4
// values each, the rule of the activation quantiser.  Workgroup-wide, with
// a barrier before (the previous chunk is consumed) and after.
template <int TT, bool DBG>
__device__ __forceinline__ void stage_qh(const FfnArgs &a, const int (&pair)[TT], int8_t *lq,
                                         float *ld) {
  const int I = a.I, nblk = I / 32;
  __syncthreads();
  for (int v = threadIdx.x; v < TT * (I / 4); v += 256) {
    const int t = v / (I / 4), k4 = v % (I / 4);
    float4 hv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (pair[t] >= 0) hv = reinterpret_cast<const float4 *>(a.h + (size_t)pair[t] * I)[k4];
    float m = fmaxf(fmaxf(fabsf(hv.x), fabsf(hv.y)), fmaxf(fabsf(hv.z), fabsf(hv.w)));
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
    const uint32_t packed = cv(hv.x) | (cv(hv.y) << 8) | (cv(hv.z) << 16) | (cv(hv.w) << 24);
    reinterpret_cast<uint32_t *>(lq + (size_t)t * I)[k4] = packed;
    if ((k4 & 7) == 0) ld[t * nblk + (k4 >> 3)] = dd;
    if (DBG && blockIdx.x == 0 && pair[t] >= 0) {
      if (a.dbg.q_h) reinterpret_cast<uint32_t *>(a.dbg.q_h + (size_t)pair[t] * I)[k4] = packed;
      if (a.dbg.d_h && (k4 & 7) == 0) a.dbg.d_h[(size_t)pair[t] * nblk + (k4 >> 3)] = dd;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ int4

// Gate/up: each wave owns GU_RPW row indices; lane l owns pieces l + 64 i.
template <int TT, int NPL, bool DBG>
__global__ void __launch_bounds__(256) k_gate_up_i4(FfnArgs a) {
  SlotInfo si;
  if (!slot_info(a, blockIdx.y, si)) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I;
  const int npieces = H / 32;
  const size_t row_b = (size_t)H / 2;
  const uint8_t *gate = si.blob;
  const uint8_t *up = si.blob + (size_t)I * row_b;
  const float *scales = reinterpret_cast<const float *>(si.blob + 3 * (size_t)I * row_b);
  const int r0 = (blockIdx.x * 4 + wv) * GU_RPW;

  for (int c0 = 0; c0 < si.n_tok; c0 += TT) {
    QBlock act[NPL][TT];
    float dq[NPL][TT];
    int pair[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) {
      int tok = 0;
      pair[t] = -1;
      if (c0 + t < si.n_tok) token_of(a, si, c0 + t, tok, pair[t]);
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
        float dd = 0.0f;
        if (pair[t] >= 0 && p < npieces) {
          const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + (size_t)tok * H + 32 * p);
          x0 = qp[0];
          x1 = qp[1];
          dd = a.d[(size_t)tok * npieces + p] * (1.0f / 16.0f);
        }
        act[i][t] = split_block(x0, x1);
        dq[i][t] = dd;
      }
    }
    uint4 wg[GU_RPW][NPL], wu[GU_RPW][NPL];
#pragma unroll
    for (int rr = 0; rr < GU_RPW; rr++) {
      const int r = r0 + rr;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        if (p < npieces) {
          wg[rr][i] = reinterpret_cast<const uint4 *>(gate + (size_t)r * row_b)[p];
          wu[rr][i] = reinterpret_cast<const uint4 *>(up + (size_t)r * row_b)[p];
        } else {
          wg[rr][i] = make_uint4(0, 0, 0, 0);
          wu[rr][i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < GU_RPW; rr++) {
      const int r = r0 + rr;
      float gacc[TT], uacc[TT];
#pragma unroll
      for (int t = 0; t < TT; t++) gacc[t] = uacc[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
#pragma unroll
        for (int t = 0; t < TT; t++) {
          const int pg = dot_int4_block16(wg[rr][i], act[i][t]);
          const int pu = dot_int4_block16(wu[rr][i], act[i][t]);
          gacc[t] = fmaf((float)pg, dq[i][t], gacc[t]);
          uacc[t] = fmaf((float)pu, dq[i][t], uacc[t]);
          if (DBG) {
            const int p = lane + 64 * i;
            if (pair[t] >= 0 && p < npieces) {
              const size_t o = ((size_t)pair[t] * I + r) * npieces + p;
              if (a.dbg.gate_dots) a.dbg.gate_dots[o] = pg >> 4;
              if (a.dbg.up_dots) a.dbg.up_dots[o] = pu >> 4;
            }
          }
        }
      }
      const float sg = scales[r], su = scales[I + r];
#pragma unroll
      for (int t = 0; t < TT; t++) {
        const float g = sg * wave_sum(gacc[t]);
        const float u = su * wave_sum(uacc[t]);
        if (lane == 0 && pair[t] >= 0) {
          const float hv = silu(g) * u;
          a.h[(size_t)pair[t] * I + r] = hv;
          if (DBG && a.dbg.h) a.dbg.h[(size_t)pair[t] * I + r] = hv;
        }
      }
    }
  }
}

// Down: prologue re-quantises h (Q8_0, same rule as the activation
// quantiser) for up to TT tokens into LDS; each wave then owns DN_RPW rows.
template <int TT, int NPL, bool DBG>
__global__ void __launch_bounds__(256) k_down_i4(FfnArgs a) {
  SlotInfo si;
  if (!slot_info(a, blockIdx.y, si)) return;
  extern __shared__ uint8_t smem[];
  const int I = a.I, H = a.H;
  int8_t *lq = reinterpret_cast<int8_t *>(smem);                    // [TT][I]
  float *ld = reinterpret_cast<float *>(smem + (size_t)TT * I);      // [TT][I/32]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int npieces = I / 32;
  const size_t row_b = (size_t)I / 2;
  const uint8_t *down = si.blob + 2 * (size_t)I * ((size_t)H / 2);
  const float *sd =
      reinterpret_cast<const float *>(si.blob + 3 * (size_t)I * ((size_t)H / 2)) + 2 * I;
  const int j0 = (blockIdx.x * 4 + wv) * DN_RPW;

  for (int c0 = 0; c0 < si.n_tok; c0 += TT) {
    int pair[TT], tok[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) {
      pair[t] = -1;
      tok[t] = 0;
      if (c0 + t < si.n_tok) token_of(a, si, c0 + t, tok[t], pair[t]);
    }
    stage_qh<TT, DBG>(a, pair, lq, ld);  // Q8_0 of h
    QBlock act[NPL][TT];
    float dq[NPL][TT];
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      const int p = lane + 64 * i;
#pragma unroll
      for (int t = 0; t < TT; t++) {
        uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
        float dd = 0.0f;
        if (p < npieces) {
          const uint4 *qp = reinterpret_cast<const uint4 *>(lq + (size_t)t * I + 32 * p);
          x0 = qp[0];
          x1 = qp[1];
          dd = ld[t * npieces + p] * (1.0f / 16.0f);
        }
        act[i][t] = split_block(x0, x1);
        dq[i][t] = dd;
      }
    }
    uint4 wd[DN_RPW][NPL];
#pragma unroll
    for (int rr = 0; rr < DN_RPW; rr++) {
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        wd[rr][i] = (p < npieces)
                        ? reinterpret_cast<const uint4 *>(down + (size_t)(j0 + rr) * row_b)[p]
                        : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int rr = 0; rr < DN_RPW; rr++) {
      const int j = j0 + rr;
      float acc[TT];
#pragma unroll
      for (int t = 0; t < TT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
#pragma unroll
        for (int t = 0; t < TT; t++) {
          const int pd = dot_int4_block16(wd[rr][i], act[i][t]);
          acc[t] = fmaf((float)pd, dq[i][t], acc[t]);
          if (DBG && a.dbg.down_dots) {
            const int p = lane + 64 * i;
            if (pair[t] >= 0 && p < npieces)
              a.dbg.down_dots[((size_t)pair[t] * H + j) * npieces + p] = pd >> 4;
          }
        }
      }
      const float s = sd[j];
#pragma unroll
      for (int t = 0; t < TT; t++) {
        const float y = s * wave_sum(acc[t]);
        if (lane == 0 && pair[t] >= 0) {
          if (si.shared)
            a.shared_out[(size_t)tok[t] * H + j] = y;
          else
            a.expert_out[(size_t)pair[t] * H + j] = y;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ int2

// Activations of one 64-code int2 piece (two Q8_0 blocks) for the field
// expansion: f[fi][j] holds bytes q[16j + fi], q[16j+4+fi], q[16j+8+fi],
// q[16j+12+fi] (the codes of field fi of word j of the weight piece).
struct QPiece2 {
  int f[4][4];
};

__device__ __forceinline__ QPiece2 split_piece2(const uint4 *qp) {
  QPiece2 r;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint4 w = qp[j];  // bytes 16j .. 16j+15
#pragma unroll
    for (int fi = 0; fi < 4; fi++) {
      const uint32_t sel_lo = (uint32_t)(fi | ((4 + fi) << 8)) | 0x0C0C0000u;
      const uint32_t a01 = __builtin_amdgcn_perm(w.y, w.x, sel_lo);  // bytes fi of w.x, w.y
      const uint32_t a23 = __builtin_amdgcn_perm(w.w, w.z, sel_lo);  // bytes fi of w.z, w.w
      r.f[fi][j] = (int)__builtin_amdgcn_perm(a23, a01, 0x05040100u);
    }
  }
  return r;
}

// 64 x exact dots of the two 32-code blocks of a 16-byte int2 piece.
__device__ __forceinline__ void dot_int2_piece64(const uint4 w, const QPiece2 &a, int &pa,
                                                 int &pb) {
  int x = 0, y = 0;
#pragma unroll
  for (int fi = 0; fi < 4; fi++) {
    x = sdot4(int2_field64(w.x, fi), a.f[fi][0], x);
    x = sdot4(int2_field64(w.y, fi), a.f[fi][1], x);
    y = sdot4(int2_field64(w.z, fi), a.f[fi][2], y);
    y = sdot4(int2_field64(w.w, fi), a.f[fi][3], y);
  }
  pa = x;
  pb = y;
}

template <int TT, int NPL, bool DBG>
__global__ void __launch_bounds__(256) k_gate_up_i2(FfnArgs a) {
  SlotInfo si;
  if (!slot_info(a, blockIdx.y, si)) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I;
  const int npieces = H / 64, nblk = H / 32;
  const size_t row_b = (size_t)H / 4;
  const uint8_t *gate = si.blob;
  const uint8_t *up = si.blob + (size_t)I * row_b;
  const float *scales = reinterpret_cast<const float *>(si.blob + 3 * (size_t)I * row_b);
  const int r0 = (blockIdx.x * 4 + wv) * GU_RPW;
  for (int c0 = 0; c0 < si.n_tok; c0 += TT) {
    QPiece2 act[NPL][TT];
    float da[NPL][TT], db[NPL][TT];
    int pair[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) {
      int tok = 0;
      pair[t] = -1;
      if (c0 + t < si.n_tok) token_of(a, si, c0 + t, tok, pair[t]);
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        uint4 z[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                      make_uint4(0, 0, 0, 0)};
        float d0 = 0.0f, d1 = 0.0f;
        if (pair[t] >= 0 && p < npieces) {
          const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + (size_t)tok * H + 64 * p);
#pragma unroll
          for (int j = 0; j < 4; j++) z[j] = qp[j];
          d0 = a.d[(size_t)tok * nblk + 2 * p] * (1.0f / 64.0f);
          d1 = a.d[(size_t)tok * nblk + 2 * p + 1] * (1.0f / 64.0f);
        }
        act[i][t] = split_piece2(z);
        da[i][t] = d0;
        db[i][t] = d1;
      }
    }
    uint4 wg[GU_RPW][NPL], wu[GU_RPW][NPL];
#pragma unroll
    for (int rr = 0; rr < GU_RPW; rr++) {
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        const bool ok = p < npieces;
        wg[rr][i] = ok ? reinterpret_cast<const uint4 *>(gate + (size_t)(r0 + rr) * row_b)[p]
                       : make_uint4(0, 0, 0, 0);
        wu[rr][i] = ok ? reinterpret_cast<const uint4 *>(up + (size_t)(r0 + rr) * row_b)[p]
                       : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int rr = 0; rr < GU_RPW; rr++) {
      const int r = r0 + rr;
      float gacc[TT], uacc[TT];
#pragma unroll
      for (int t = 0; t < TT; t++) gacc[t] = uacc[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
#pragma unroll
        for (int t = 0; t < TT; t++) {
          int ga, gb, ua, ub;
          dot_int2_piece64(wg[rr][i], act[i][t], ga, gb);
          dot_int2_piece64(wu[rr][i], act[i][t], ua, ub);
          gacc[t] = fmaf((float)ga, da[i][t], gacc[t]);
          gacc[t] = fmaf((float)gb, db[i][t], gacc[t]);
          uacc[t] = fmaf((float)ua, da[i][t], uacc[t]);
          uacc[t] = fmaf((float)ub, db[i][t], uacc[t]);
          if (DBG) {
            const int p = lane + 64 * i;
            if (pair[t] >= 0 && p < npieces) {
              const size_t o = ((size_t)pair[t] * I + r) * nblk + 2 * p;
              if (a.dbg.gate_dots) {
                a.dbg.gate_dots[o] = ga >> 6;
                a.dbg.gate_dots[o + 1] = gb >> 6;
              }
              if (a.dbg.up_dots) {
                a.dbg.up_dots[o] = ua >> 6;
                a.dbg.up_dots[o + 1] = ub >> 6;
              }
            }
          }
        }
      }
      const float sg = scales[r], su = scales[I + r];
#pragma unroll
      for (int t = 0; t < TT; t++) {
        const float g = sg * wave_sum(gacc[t]);
        const float u = su * wave_sum(uacc[t]);
        if (lane == 0 && pair[t] >= 0) {
          const float hv = silu(g) * u;
          a.h[(size_t)pair[t] * I + r] = hv;
          if (DBG && a.dbg.h) a.dbg.h[(size_t)pair[t] * I + r] = hv;
        }
      }
    }
  }
}

template <int TT, int NPL, bool DBG>
__global__ void __launch_bounds__(256) k_down_i2(FfnArgs a) {
  SlotInfo si;
  if (!slot_info(a, blockIdx.y, si)) return;
  extern __shared__ uint8_t smem[];
  const int I = a.I, H = a.H;
  int8_t *lq = reinterpret_cast<int8_t *>(smem);
  float *ld = reinterpret_cast<float *>(smem + (size_t)TT * I);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int npieces = I / 64, nblk = I / 32;
  const size_t row_b = (size_t)I / 4;
  const uint8_t *down = si.blob + 2 * (size_t)I * ((size_t)H / 4);
  const float *sd =
      reinterpret_cast<const float *>(si.blob + 3 * (size_t)I * ((size_t)H / 4)) + 2 * I;
  const int j0 = (blockIdx.x * 4 + wv) * DN_RPW;
  for (int c0 = 0; c0 < si.n_tok; c0 += TT) {
    int pair[TT], tok[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) {
      pair[t] = -1;
      tok[t] = 0;
      if (c0 + t < si.n_tok) token_of(a, si, c0 + t, tok[t], pair[t]);
    }
    stage_qh<TT, DBG>(a, pair, lq, ld);  // Q8_0 of h
    QPiece2 act[NPL][TT];
    float da[NPL][TT], db[NPL][TT];
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      const int p = lane + 64 * i;
#pragma unroll
      for (int t = 0; t < TT; t++) {
        uint4 z[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                      make_uint4(0, 0, 0, 0)};
        float d0 = 0.0f, d1 = 0.0f;
        if (p < npieces) {
          const uint4 *qp = reinterpret_cast<const uint4 *>(lq + (size_t)t * I + 64 * p);
#pragma unroll
          for (int j = 0; j < 4; j++) z[j] = qp[j];
          d0 = ld[t * nblk + 2 * p] * (1.0f / 64.0f);
          d1 = ld[t * nblk + 2 * p + 1] * (1.0f / 64.0f);
        }
        act[i][t] = split_piece2(z);
        da[i][t] = d0;
        db[i][t] = d1;
      }
    }
    uint4 wd[DN_RPW][NPL];
#pragma unroll
    for (int rr = 0; rr < DN_RPW; rr++) {
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        wd[rr][i] = (p < npieces)
                        ? reinterpret_cast<const uint4 *>(down + (size_t)(j0 + rr) * row_b)[p]
                        : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int rr = 0; rr < DN_RPW; rr++) {
      const int j = j0 + rr;
      float acc[TT];
#pragma unroll
      for (int t = 0; t < TT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
#pragma unroll
        for (int t = 0; t < TT; t++) {
          int pa, pb;
          dot_int2_piece64(wd[rr][i], act[i][t], pa, pb);
          acc[t] = fmaf((float)pa, da[i][t], acc[t]);
          acc[t] = fmaf((float)pb, db[i][t], acc[t]);
          if (DBG && a.dbg.down_dots) {
            const int p = lane + 64 * i;
            if (pair[t] >= 0 && p < npieces) {
              const size_t o = ((size_t)pair[t] * H + j) * nblk + 2 * p;
              a.dbg.down_dots[o] = pa >> 6;
              a.dbg.down_dots[o + 1] = pb >> 6;
            }
          }
        }
      }
      const float s = sd[j];
#pragma unroll
      for (int t = 0; t < TT; t++) {
        const float y = s * wave_sum(acc[t]);
        if (lane == 0 && pair[t] >= 0) {
          if (si.shared)
            a.shared_out[(size_t)tok[t] * H + j] = y;
          else
            a.expert_out[(size_t)pair[t] * H + j] = y;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ FP8

// FP8 E4M3 experts with one fp32 scale per 128x128 block ("Comment exécuter
// un réseau de neurones de 744 milliards de paramètres…", section "Modèles
// supportés": a supported model runs on fp4/fp8 weights; "Show HN…",
// converter item: its FP8 checkpoints carry 128x128 block scales).  A lane
// takes whole 32-code blocks (32 bytes); the codes become the exact integers
// 512 x value (gfx950's OCP E4M3 conversion, scaled by 512: at most 18
// bits) and meet the block's int8 activations in 24-bit integer
// multiply-adds, so each block dot P9 = sum 512 fp8(c) q is exact; the
// float epilogue per block is acc += P9 * (d * S) with S the block's
// 128x128 scale, and the row is scaled by 1/512 at the end.

// P9 of one block: codes w0, w1 (32 bytes) against the block's activation
// bytes x0, x1 (kept packed; each byte is sign-extended where it is used, so
// a lane holds 8 activation words per block rather than 32).
__device__ __forceinline__ int dot_fp8_block(const uint4 w0, const uint4 w1, const uint4 x0,
                                             const uint4 x1) {
  const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  const uint32_t x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  int acc = 0;
#pragma unroll
  for (int j = 0; j < 8; j++) acc = dot_fp8_word(w[j], x[j], acc);
  return acc;
}


// Gate/up: one gate/up row pair per wave, lane l takes blocks l + 64 i; the
// weights stay in registers while the slot's tokens go through them.
template <int NPL, bool DBG>
__global__ void __launch_bounds__(256) k_gate_up_f8(FfnArgs a) {
  SlotInfo si;
  if (!slot_info(a, blockIdx.y, si)) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I, nblk = H / 32, nsb = H / 128;
  const uint8_t *gate = si.blob, *up = si.blob + (size_t)I * H;
  const float *bs = reinterpret_cast<const float *>(si.blob + 3 * (size_t)I * H);
  const size_t nbs = (size_t)(I / 128) * nsb;
  const int r = blockIdx.x * 4 + wv;
  const float *sgr = bs + (size_t)(r / 128) * nsb, *sur = bs + nbs + (size_t)(r / 128) * nsb;
  uint4 wg[NPL][2], wu[NPL][2];
  float sg[NPL], su[NPL];
#pragma unroll
  for (int i = 0; i < NPL; i++) {
    const int p = lane + 64 * i;
    const bool ok = p < nblk;
    const uint4 *gp = reinterpret_cast<const uint4 *>(gate + (size_t)r * H + 32 * (ok ? p : 0));
    const uint4 *upp = reinterpret_cast<const uint4 *>(up + (size_t)r * H + 32 * (ok ? p : 0));
    wg[i][0] = gp[0];
    wg[i][1] = gp[1];
    wu[i][0] = upp[0];
    wu[i][1] = upp[1];
    sg[i] = ok ? sgr[p / 4] : 0.0f;
    su[i] = ok ? sur[p / 4] : 0.0f;
  }
  for (int c = 0; c < si.n_tok; c++) {
    int tok, pair;
    token_of(a, si, c, tok, pair);
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      opaque_words(wg[i][0]);
      opaque_words(wg[i][1]);
      opaque_words(wu[i][0]);
      opaque_words(wu[i][1]);
    }
    float gacc = 0.0f, uacc = 0.0f;
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      const int p = lane + 64 * i;
      const bool ok = p < nblk;
      const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + (size_t)tok * H + 32 * (ok ? p : 0));
      const uint4 x0 = qp[0], x1 = qp[1];
      const float dd = ok ? a.d[(size_t)tok * nblk + p] : 0.0f;
      const int pg = dot_fp8_block(wg[i][0], wg[i][1], x0, x1);
      const int pu = dot_fp8_block(wu[i][0], wu[i][1], x0, x1);
      gacc = fmaf((float)pg, dd * sg[i], gacc);
      uacc = fmaf((float)pu, dd * su[i], uacc);
      if (DBG && ok) {
        const size_t o = ((size_t)pair * I + r) * nblk + p;
        if (a.dbg.gate_dots) a.dbg.gate_dots[o] = pg;
        if (a.dbg.up_dots) a.dbg.up_dots[o] = pu;
      }
    }
    const float g = wave_sum(gacc) * (1.0f / 512.0f);
    const float u = wave_sum(uacc) * (1.0f / 512.0f);
    if (lane == 0) {
      const float hv = silu(g) * u;
      a.h[(size_t)pair * I + r] = hv;
      if (DBG && a.dbg.h) a.dbg.h[(size_t)pair * I + r] = hv;
    }
  }
}

// Down: Q8_0 of h for TT pairs into LDS (stage_qh), then DN_RPW rows per
// wave, lane l taking blocks l + 64 i of each row.
template <int TT, int NPL, bool DBG>
__global__ void __launch_bounds__(256) k_down_f8(FfnArgs a) {
  SlotInfo si;
  if (!slot_info(a, blockIdx.y, si)) return;
  extern __shared__ uint8_t smem[];
  const int I = a.I, H = a.H, nblk = I / 32, nsb = I / 128;
  int8_t *lq = reinterpret_cast<int8_t *>(smem);                // [TT][I]
  float *ld = reinterpret_cast<float *>(smem + (size_t)TT * I);  // [TT][I/32]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint8_t *down = si.blob + 2 * (size_t)I * H;
  const float *bs = reinterpret_cast<const float *>(si.blob + 3 * (size_t)I * H) +
                    2 * (size_t)(I / 128) * (H / 128);
  const int j0 = (blockIdx.x * 4 + wv) * DN_RPW;
  uint4 wd[DN_RPW][NPL][2];
  float sd[DN_RPW][NPL];
#pragma unroll
  for (int rr = 0; rr < DN_RPW; rr++)
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      const int p = lane + 64 * i, j = j0 + rr;
      const bool ok = p < nblk;
      const uint4 *dp = reinterpret_cast<const uint4 *>(down + (size_t)j * I + 32 * (ok ? p : 0));
      wd[rr][i][0] = dp[0];
      wd[rr][i][1] = dp[1];
      sd[rr][i] = ok ? bs[(size_t)(j / 128) * nsb + p / 4] : 0.0f;
    }
  for (int c0 = 0; c0 < si.n_tok; c0 += TT) {
    int pair[TT], tok[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) {
      pair[t] = -1;
      tok[t] = 0;
      if (c0 + t < si.n_tok) token_of(a, si, c0 + t, tok[t], pair[t]);
    }
    stage_qh<TT, DBG>(a, pair, lq, ld);  // Q8_0 of h
    float acc[DN_RPW][TT];
#pragma unroll
    for (int rr = 0; rr < DN_RPW; rr++) {
#pragma unroll
      for (int t = 0; t < TT; t++) acc[rr][t] = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        opaque_words(wd[rr][i][0]);
        opaque_words(wd[rr][i][1]);
      }
    }
#pragma unroll
    for (int t = 0; t < TT; t++) {
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        const bool ok = p < nblk;
        const uint4 *qp = reinterpret_cast<const uint4 *>(lq + (size_t)t * I + 32 * (ok ? p : 0));
        const uint4 x0 = qp[0], x1 = qp[1];
        const float dd = ok ? ld[t * nblk + p] : 0.0f;
#pragma unroll
        for (int rr = 0; rr < DN_RPW; rr++) {
          const int pd = dot_fp8_block(wd[rr][i][0], wd[rr][i][1], x0, x1);
          acc[rr][t] = fmaf((float)pd, dd * sd[rr][i], acc[rr][t]);
          if (DBG && a.dbg.down_dots && pair[t] >= 0 && ok)
            a.dbg.down_dots[((size_t)pair[t] * H + j0 + rr) * nblk + p] = pd;
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < DN_RPW; rr++) {
      const int j = j0 + rr;
#pragma unroll
      for (int t = 0; t < TT; t++) {
        const float y = wave_sum(acc[rr][t]) * (1.0f / 512.0f);
        if (lane == 0 && pair[t] >= 0) {
          if (si.shared)
            a.shared_out[(size_t)tok[t] * H + j] = y;
          else
            a.expert_out[(size_t)pair[t] * H + j] = y;
        }
      }
    }
  }
}

template <int TT, int NG, int ND, bool DBG>
static void launch_f8_tt(const FfnArgs &a, int n_slots, hipStream_t st, const moe_events *ev) {
  const size_t lds = (size_t)TT * a.I + sizeof(float) * (size_t)TT * (a.I / 32);
  launch_k(k_gate_up_f8<NG, DBG>, dim3(a.I / 4, n_slots), dim3(256), 0, st,
           stage_ev(ev, MOE_STAGE_GATE_UP), a);
  launch_k(k_down_f8<TT, ND, DBG>, dim3(a.H / (4 * DN_RPW), n_slots), dim3(256), (uint32_t)lds,
           st, stage_ev(ev, MOE_STAGE_DOWN), a);
}

template <int TT, bool DBG>
static void launch_f8_shape(const FfnArgs &a, int n_slots, hipStream_t st,
                            const moe_events *ev) {
  const int ng = (a.H / 32 + 63) / 64, nd = (a.I / 32 + 63) / 64;
  if (ng <= 1 && nd <= 1) launch_f8_tt<TT, 1, 1, DBG>(a, n_slots, st, ev);
  else if (ng <= 2 && nd <= 1) launch_f8_tt<TT, 2, 1, DBG>(a, n_slots, st, ev);
  else if (ng <= 3 && nd <= 1) launch_f8_tt<TT, 3, 1, DBG>(a, n_slots, st, ev);
  else if (ng <= 4 && nd <= 1) launch_f8_tt<TT, 4, 1, DBG>(a, n_slots, st, ev);
  else launch_f8_tt<TT, 4, 2, DBG>(a, n_slots, st, ev);
}

bool f8_supported(const FfnArgs &a) {
  return a.H % 128 == 0 && a.I % 128 == 0 && a.H / 32 <= 256 && a.I / 32 <= 128 &&
         a.H % (4 * DN_RPW) == 0;
}

void launch_ffn_f8(const FfnArgs &a, hipStream_t st, const moe_events *ev) {
  const int n_slots = a.n_shared + (a.T * a.K < a.E ? a.T * a.K : a.E);
  const bool dbg = a.dbg.gate_dots || a.dbg.up_dots || a.dbg.h || a.dbg.q_h || a.dbg.d_h ||
                   a.dbg.down_dots;
  const int tt = a.T <= 1 ? 1 : (a.T <= 2 ? 2 : 4);
  if (dbg) {
    if (tt == 1) launch_f8_shape<1, true>(a, n_slots, st, ev);
    else if (tt == 2) launch_f8_shape<2, true>(a, n_slots, st, ev);
    else launch_f8_shape<4, true>(a, n_slots, st, ev);
  } else {
    if (tt == 1) launch_f8_shape<1, false>(a, n_slots, st, ev);
    else if (tt == 2) launch_f8_shape<2, false>(a, n_slots, st, ev);
    else launch_f8_shape<4, false>(a, n_slots, st, ev);
  }
}

// ------------------------------------------------------------------ launch

template <int TT, int NG, int ND, bool DBG>
static void launch_tt(const FfnArgs &a, int n_slots, hipStream_t st, const moe_events *ev) {
  const Ev eg = stage_ev(ev, MOE_STAGE_GATE_UP), ed = stage_ev(ev, MOE_STAGE_DOWN);
  const dim3 g_gu(a.I / (4 * GU_RPW), n_slots);
  const dim3 g_dn(a.H / (4 * DN_RPW), n_slots);
  const size_t lds = (size_t)TT * a.I + sizeof(float) * (size_t)TT * (a.I / 32);
  if (a.wbits == 4) {
    launch_k(k_gate_up_i4<TT, NG, DBG>, g_gu, dim3(256), 0, st, eg, a);
    launch_k(k_down_i4<TT, ND, DBG>, g_dn, dim3(256), (uint32_t)lds, st, ed, a);
  } else {
    launch_k(k_gate_up_i2<TT, NG, DBG>, g_gu, dim3(256), 0, st, eg, a);
    launch_k(k_down_i2<TT, ND, DBG>, g_dn, dim3(256), (uint32_t)lds, st, ed, a);
  }
}

// pieces per lane: gate/up rows have H/32 (int4) or H/64 (int2) 16-byte
// pieces, down rows I/32 or I/64; template instances cover up to 4 and 2.
template <int TT, bool DBG>
static void launch_shape(const FfnArgs &a, int n_slots, hipStream_t st, const moe_events *ev) {
  const int per = a.wbits == 4 ? 32 : 64;
  const int ng = (a.H / per + 63) / 64, nd = (a.I / per + 63) / 64;
  if (ng <= 1 && nd <= 1) launch_tt<TT, 1, 1, DBG>(a, n_slots, st, ev);
  else if (ng <= 2 && nd <= 1) launch_tt<TT, 2, 1, DBG>(a, n_slots, st, ev);
  else if (ng <= 3 && nd <= 1) launch_tt<TT, 3, 1, DBG>(a, n_slots, st, ev);
  else if (ng <= 4 && nd <= 1) launch_tt<TT, 4, 1, DBG>(a, n_slots, st, ev);
  else launch_tt<TT, 4, 2, DBG>(a, n_slots, st, ev);
}

void launch_ffn_gemv(const FfnArgs &a, hipStream_t st, const moe_events *ev) {
  const int n_slots = a.n_shared + (a.T * a.K < a.E ? a.T * a.K : a.E);
  const bool dbg = a.dbg.gate_dots || a.dbg.up_dots || a.dbg.h || a.dbg.q_h || a.dbg.d_h ||
                   a.dbg.down_dots;
  const int tt = a.T <= 1 ? 1 : (a.T <= 2 ? 2 : (a.T <= 4 ? 4 : 8));
  if (dbg) {
    if (tt == 1) launch_shape<1, true>(a, n_slots, st, ev);
    else if (tt == 2) launch_shape<2, true>(a, n_slots, st, ev);
    else if (tt == 4) launch_shape<4, true>(a, n_slots, st, ev);
    else launch_shape<8, true>(a, n_slots, st, ev);
  } else {
    if (tt == 1) launch_shape<1, false>(a, n_slots, st, ev);
    else if (tt == 2) launch_shape<2, false>(a, n_slots, st, ev);
    else if (tt == 4) launch_shape<4, false>(a, n_slots, st, ev);
    else launch_shape<8, false>(a, n_slots, st, ev);
  }
}

}  // namespace moe

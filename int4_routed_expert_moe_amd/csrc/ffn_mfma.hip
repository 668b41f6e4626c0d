// Expert FFNs for large batches (prefill): grouped int4 x int8 GEMMs on the
// matrix cores ("Show HN: 遅いコンピュータで GLM 5.2 を実行する", section
// 実装済みの主な機能: packed int4 weights with per-row scales dequantised on
// use, integer-dot kernels on Q8_0-style int8 activations, batch-union MoE).
//
// Same arithmetic as the GEMV path: for every (token, row) of an expert,
//   acc = sum_b d[t,b] * P[t,r,b],  P = exact int32 dot of block b (32 codes)
// then g = sg[r]*acc (and u), h = silu(g)*u, Q8_0(h), and the down projection
// y = sd[j] * sum_b d_h[b] * P_down[j,b].
//
// One v_mfma_i32_16x16x32_i8 computes the 16x16 block dots of one Q8_0 block
// exactly (K = 32 = the block), so the per-block scales are applied by a VALU
// fix-up (convert, fused multiply-add) after every MFMA.  int4 codes enter
// the MFMA as 16 x code (the low/high nibble split), with the 1/16 folded
// into the activation scale; the split reorders k inside each group of 8,
// and the activations staged in LDS are reordered the same way.  int8 codes
// (the same format with 8-bit codes) enter as they are; int2 codes (the small-
// batch down tiles only) as 64 x code, in the field order of the activations
// the small-batch gate/up kernel writes, with 1/64 folded into the scale.
//
// Work items are (expert, 64-token tile) pairs from a tile list; a
// workgroup computes 64 rows x 64 tokens of one work item (gate and up
// together, so SwiGLU and the Q8_0 of h happen in its epilogue).  The
// small-batch path's down projection (4..16 tokens) uses the same K loop on
// (64-row tile, expert slot) workgroups read from its slot table, staging 16
// token rows.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {

namespace mf {
constexpr int NT = TILE_T;          // tokens per tile
constexpr int RT = 64;              // rows per workgroup
constexpr int CB = 8;               // Q8_0 blocks per K chunk (256 k)
constexpr int BSTR = CB * 32 + 16;  // LDS bytes per activation row (padded)
// LDS bytes per weight row of a chunk (padded): int4 16 B per block, int8 32
// B, int2 8 B
template <int WB>
constexpr int astr() { return WB == 8 ? CB * 32 + 8 : WB == 2 ? CB * 8 + 4 : CB * 16 + 4; }
}  // namespace mf


// --------------------------------------------------------------- tile list

// tiles[i] = {expert (E = shared), first list position, token count}.  Routed
// tokens of expert e are perm[offsets[e] ..]; the shared expert takes tokens
// 0..T-1 in order.  One workgroup of 256 threads.
__global__ void __launch_bounds__(256) k_mfma_tiles(int E, int T, int n_shared,
                                                    const int32_t *offsets, int4 *tiles,
                                                    int32_t *n_tiles) {
  __shared__ int wt[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int c[4], loc = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {  // 4 consecutive experts per thread (E <= 1024)
    const int e = tid * 4 + j;
    const int n = e < E ? offsets[e + 1] - offsets[e] : 0;
    c[j] = (n + mf::NT - 1) / mf::NT;
    loc += c[j];
  }
  int x = loc;  // inclusive scan over the block
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wt[wv] = x;
  __syncthreads();
  int pre = x - loc, total = 0;
  for (int w = 0; w < 4; w++) {
    pre += w < wv ? wt[w] : 0;
    total += wt[w];
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = tid * 4 + j;
    if (e < E) {
      const int n = offsets[e + 1] - offsets[e];
      for (int i = 0; i < c[j]; i++)
        tiles[pre + i] = make_int4(e, offsets[e] + i * mf::NT, min(mf::NT, n - i * mf::NT), 0);
    }
    pre += c[j];
  }
  const int ns = n_shared ? (T + mf::NT - 1) / mf::NT : 0;
  for (int i = tid; i < ns; i += 256)
    tiles[total + i] = make_int4(E, i * mf::NT, min(mf::NT, T - i * mf::NT), 0);
  if (tid == 0) *n_tiles = total + ns;
}

// ---------------------------------------------------------------- helpers





// A fragment of one 32-code block: lane (m, g) holds codes 8g..8g+7 of row m
// -- int4: as 16 x code, even codes first (from 4 bytes); MXFP4: as 2 x the
// FP4 value, even codes first; int8: the 8 bytes; int2: codes g + 4 i
// (i = 0..7, field g of each of the block's 8 bytes) as 64 x code, the order
// in which the small-batch gate/up kernel writes Q8_0(h) for int2 (bytes
// 16 g + 8 (b & 1) .. + 7 of each 64-code piece).
template <int WB>
__device__ __forceinline__ long a_frag(const uint8_t *row, int b, int g) {
  if constexpr (WB == 8) {
    return *reinterpret_cast<const long *>(row + b * 32 + g * 8);
  } else if constexpr (WB == 2) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(row + b * 8);
    const uint32_t lo = ((w[0] >> (2 * g)) & 0x03030303u) << 6;
    const uint32_t hi = ((w[1] >> (2 * g)) & 0x03030303u) << 6;
    return (long)lo | ((long)hi << 32);
  } else if constexpr (WB == WB_MX) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(row + b * 16 + g * 4);
    return (long)(uint32_t)mx_lanes(w, 0) | ((long)(uint32_t)mx_lanes(w, 4) << 32);
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(row + b * 16 + g * 4);
    return (long)(uint32_t)lo16(w) | ((long)(uint32_t)hi16(w) << 32);
  }
}

// Stage one K chunk of activations: rows = tokens (64), CB blocks of 32
// int8 and their scales (for int4 and MXFP4 weights: reordered per 8 like
// the nibble split, and the scales / 16 or / 2).  The loads are
// unconditional (a block past the row reads the row's last block, a token
// past n the list's entry, which always names a valid row) and a position
// outside the tile gets a zero scale when the chunk is stored: a load inside
// a branch would make the compiler wait for it (and for every load before
// it) on the spot, ahead of the MFMAs it is meant to overlap.
template <int TR>
struct ActChunk {
  static constexpr int NV = TR * 16 / 256;          // 16-byte pieces per thread
  static constexpr int ND = (TR * mf::CB + 255) / 256;  // block scales per thread
  uint4 v[NV];  // TR tokens x 16 pieces
  float d[ND];  // TR tokens x 8 block scales, as loaded
};

template <int WB, int TR>
__device__ __forceinline__ void load_act_chunk(const int8_t *q, const float *d, int row_len,
                                               const int *tokl, int n, int c, int nblk,
                                               ActChunk<TR> &r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < ActChunk<TR>::NV; u++) {
    const int i = tid + 256 * u, tok_i = i >> 4, piece = i & 15;  // 16-byte piece
    const int blk = min(c * mf::CB + (piece >> 1), nblk - 1);
    r.v[u] = gload<uint4>(reinterpret_cast<const uint8_t *>(q),
                          (size_t)tokl[tok_i] * row_len + (size_t)blk * 32 + (piece & 1) * 16);
  }
#pragma unroll
  for (int u = 0; u < ActChunk<TR>::ND; u++) {
    const int i = min(tid + 256 * u, TR * mf::CB - 1), tok_i = i >> 3, b = i & 7;
    const int blk = min(c * mf::CB + b, nblk - 1);
    r.d[u] = gload<float>(reinterpret_cast<const uint8_t *>(d),
                          4 * ((size_t)tokl[tok_i] * (row_len / 32) + blk));
  }
}

template <int WB, int TR>
__device__ __forceinline__ void store_act_chunk(const ActChunk<TR> &r, uint8_t *bs, float *ds,
                                                int n, int c, int nblk) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < ActChunk<TR>::NV; u++) {
    const int i = tid + 256 * u, tok_i = i >> 4, piece = i & 15;
    if constexpr (WB == 8 || WB == 2) {  // int2: already in its fragment order
      *reinterpret_cast<uint4 *>(bs + tok_i * mf::BSTR + piece * 16) = r.v[u];
    } else {
      uint2 *dst = reinterpret_cast<uint2 *>(bs + tok_i * mf::BSTR + piece * 16);
      dst[0] = even_odd8(r.v[u].x, r.v[u].y);
      dst[1] = even_odd8(r.v[u].z, r.v[u].w);
    }
  }
#pragma unroll
  for (int u = 0; u < ActChunk<TR>::ND; u++) {
    const int i = tid + 256 * u, tok_i = i >> 3, b = i & 7;
    const bool ok = tok_i < n && c * mf::CB + b < nblk;
    if (i < TR * mf::CB)
      ds[tok_i * mf::CB + b] =
          ok ? r.d[u] * (WB == 8 ? 1.0f : WB == WB_MX ? 0.5f : WB == 2 ? 0.015625f : 0.0625f)
             : 0.0f;
  }
}

// Stage one K chunk of NM weight matrices: 64 rows x CB blocks x (4 bits)
// bytes, as 16-byte pieces (PPR per row); MXFP4 also the 64 x CB scale bytes
// (two per thread).
template <int NM, int WB>
struct WChunk {
  static constexpr int PPR = mf::CB * code_bits<WB>() / 4;  // pieces per row: 4-bit 8, int8 16
  uint4 v[NM * PPR / 4];                                     // 64 rows x PPR pieces / 256 threads
  uint32_t sc[NM];                                           // MXFP4: 2 scale bytes
};

// NT: non-temporal loads, for weights read once per launch (the slot-table
// down kernel of the small-batch path); prefill tiles of one expert re-read
// its rows, which ordinary loads keep in the caches.
template <int NM, int WB, bool NT>
__device__ __forceinline__ void load_w_chunk(const uint8_t *const *mat,
                                             const uint8_t *const *scl, size_t row_b, int r0,
                                             int c, int nblk, WChunk<NM, WB> &r) {
  constexpr int PPR = WChunk<NM, WB>::PPR, PER = PPR / 4, CW = code_bits<WB>();
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 0; m < NM; m++) {
#pragma unroll
    for (int u = 0; u < PER; u++) {
      const int i = tid + 256 * u, row = i / PPR, pc = i % PPR;
      // a block past the row: the row's last 16 bytes (its activations have
      // zero scales), so that the load is unconditional
      const int blk = c * mf::CB + pc * 16 / (4 * CW);
      const size_t off = blk < nblk ? (size_t)c * mf::CB * 4 * CW + pc * 16 : row_b - 16;
      r.v[m * PER + u] = NT ? gload_stream(mat[m], (size_t)(r0 + row) * row_b + off)
                            : gload<uint4>(mat[m], (size_t)(r0 + row) * row_b + off);
    }
    if constexpr (WB == WB_MX) {  // row tid / 4, blocks 2 (tid % 4), +1 of the chunk
      const int row = tid >> 2, blk = min(c * mf::CB + 2 * (tid & 3), nblk - 2);
      r.sc[m] = gload<uint16_t>(scl[m], (size_t)(r0 + row) * nblk + blk);
    }
  }
}

// wsl (MXFP4): the chunk's block scales as floats, [NM][CB][64 rows].
template <int NM, int WB>
__device__ __forceinline__ void store_w_chunk(const WChunk<NM, WB> &r, uint8_t *as, float *wsl) {
  constexpr int PPR = WChunk<NM, WB>::PPR, PER = PPR / 4, AS = mf::astr<WB>();
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 0; m < NM; m++) {
    if constexpr (WB == WB_MX) {
      const int row = tid >> 2, b = 2 * (tid & 3);
      wsl[(m * mf::CB + b) * mf::RT + row] = e8m0_float(r.sc[m] & 0xFFu);
      wsl[(m * mf::CB + b + 1) * mf::RT + row] = e8m0_float(r.sc[m] >> 8);
    }
#pragma unroll
    for (int u = 0; u < PER; u++) {
      const int i = tid + 256 * u, row = i / PPR, pc = i % PPR;
      uint8_t *dst = as + (size_t)m * mf::RT * AS + row * AS + pc * 16;
      const uint4 v = r.v[m * PER + u];
      if constexpr (WB == 8) {  // rows 8-byte aligned
        reinterpret_cast<uint2 *>(dst)[0] = make_uint2(v.x, v.y);
        reinterpret_cast<uint2 *>(dst)[1] = make_uint2(v.z, v.w);
      } else {  // rows 4-byte aligned
        uint32_t *d32 = reinterpret_cast<uint32_t *>(dst);
        d32[0] = v.x;
        d32[1] = v.y;
        d32[2] = v.z;
        d32[3] = v.w;
      }
    }
  }
}

// The K loop shared by both kernels: NM weight matrices (gate+up: 2, down:
// 1) times the tile's activations; acc[m][s][i] = sum_b d*P for matrix m,
// token sub-tile s (16 tokens, s < NS: the sub-tiles that hold tokens, fixed
// per workgroup so the loop body has no branches), row 16 wv + 4 g + i.  DBG: raw block dots of
// matrix m go to dots[m] at ((pair * R + row) * nblk + block).
template <int NM, bool DBG, int NS, int WB, bool NT, int TR>
__device__ void mfma_kloop(const uint8_t *const *mat, const uint8_t *const *scl, size_t row_b,
                           int r0, const int8_t *q, const float *d, int row_len, const int *tokl,
                           const int *pairl, int n, int nblk, uint8_t *bs, float *ds, uint8_t *as,
                           float *wsl, float (&acc)[NM][4][4], int32_t *const *dots, int R) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int m = 0; m < NM; m++)
#pragma unroll
    for (int s = 0; s < 4; s++)
#pragma unroll
      for (int i = 0; i < 4; i++) acc[m][s][i] = 0.0f;
  const int nchunk = (nblk + mf::CB - 1) / mf::CB;
  constexpr int AS = mf::astr<WB>();
  static_assert(16 * NS <= TR, "token sub-tiles within the staged rows");
  ActChunk<TR> ac;
  WChunk<NM, WB> wc;
  load_act_chunk<WB, TR>(q, d, row_len, tokl, n, 0, nblk, ac);
  load_w_chunk<NM, WB, NT>(mat, scl, row_b, r0, 0, nblk, wc);
  for (int c = 0; c < nchunk; c++) {
    __syncthreads();  // the previous chunk is consumed
    store_act_chunk<WB, TR>(ac, bs, ds, n, c, nblk);
    store_w_chunk<NM, WB>(wc, as, wsl);
    __syncthreads();
    if (c + 1 < nchunk) {  // next chunk in flight during this one's MFMAs
      load_act_chunk<WB, TR>(q, d, row_len, tokl, n, c + 1, nblk, ac);
      load_w_chunk<NM, WB, NT>(mat, scl, row_b, r0, c + 1, nblk, wc);
    }
    const int nb = min(mf::CB, nblk - c * mf::CB);
    for (int b = 0; b < nb; b++) {
      long af[NM];
#pragma unroll
      for (int m = 0; m < NM; m++)
        af[m] = a_frag<WB>(as + (size_t)m * mf::RT * AS + (wv * 16 + m16) * AS, b, g);
      float4 wsv[NM];  // MXFP4: block scales of this lane's 4 rows
#pragma unroll
      for (int m = 0; m < NM; m++)
        wsv[m] = WB == WB_MX ? *reinterpret_cast<const float4 *>(
                                   wsl + (m * mf::CB + b) * mf::RT + wv * 16 + g * 4)
                             : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
#pragma unroll
      for (int s = 0; s < NS; s++) {  // only the sub-tiles that hold tokens
        const int col = s * 16 + m16;
        const int bo = WB == 2 ? (b >> 1) * 64 + g * 16 + (b & 1) * 8 : b * 32 + g * 8;
        const long bf = *reinterpret_cast<const long *>(bs + col * mf::BSTR + bo);
        const float dd = ds[col * mf::CB + b];
#pragma unroll
        for (int m = 0; m < NM; m++) {
          const v4i z = {0, 0, 0, 0};
          const v4i p = __builtin_amdgcn_mfma_i32_16x16x32_i8(af[m], bf, z, 0, 0, 0);
          if constexpr (WB == WB_MX) {
            acc[m][s][0] = fmaf(dd * wsv[m].x, (float)p[0], acc[m][s][0]);
            acc[m][s][1] = fmaf(dd * wsv[m].y, (float)p[1], acc[m][s][1]);
            acc[m][s][2] = fmaf(dd * wsv[m].z, (float)p[2], acc[m][s][2]);
            acc[m][s][3] = fmaf(dd * wsv[m].w, (float)p[3], acc[m][s][3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; i++) acc[m][s][i] = fmaf(dd, (float)p[i], acc[m][s][i]);
          }
          if (DBG && dots[m] && col < n) {
            const int blk = c * mf::CB + b;
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int row = r0 + wv * 16 + g * 4 + i;
              dots[m][((size_t)pairl[col] * R + row) * nblk + blk] =
                  WB == 4 ? p[i] >> 4 : WB == 2 ? p[i] >> 6 : p[i];
            }
          }
        }
      }
    }
  }
}

// mfma_kloop with the sub-tile count of n tokens chosen once; TR token rows
// are staged per chunk (16 when the work item never holds more tokens).
template <int NM, bool DBG, int WB, bool NT = false, int TR = mf::NT>
__device__ void mfma_kloop_n(const uint8_t *const *mat, const uint8_t *const *scl, size_t row_b,
                             int r0, const int8_t *q, const float *d, int row_len,
                             const int *tokl, const int *pairl, int n, int nblk, uint8_t *bs,
                             float *ds, uint8_t *as, float *wsl, float (&acc)[NM][4][4],
                             int32_t *const *dots, int R) {
  if constexpr (TR == 16) {
    mfma_kloop<NM, DBG, 1, WB, NT, TR>(mat, scl, row_b, r0, q, d, row_len, tokl, pairl, n, nblk,
                                       bs, ds, as, wsl, acc, dots, R);
  } else {
    switch ((n + 15) / 16) {
      case 1:
        mfma_kloop<NM, DBG, 1, WB, NT, TR>(mat, scl, row_b, r0, q, d, row_len, tokl, pairl, n,
                                           nblk, bs, ds, as, wsl, acc, dots, R);
        break;
      case 2:
        mfma_kloop<NM, DBG, 2, WB, NT, TR>(mat, scl, row_b, r0, q, d, row_len, tokl, pairl, n,
                                           nblk, bs, ds, as, wsl, acc, dots, R);
        break;
      case 3:
        mfma_kloop<NM, DBG, 3, WB, NT, TR>(mat, scl, row_b, r0, q, d, row_len, tokl, pairl, n,
                                           nblk, bs, ds, as, wsl, acc, dots, R);
        break;
      default:
        mfma_kloop<NM, DBG, 4, WB, NT, TR>(mat, scl, row_b, r0, q, d, row_len, tokl, pairl, n,
                                           nblk, bs, ds, as, wsl, acc, dots, R);
    }
  }
}

constexpr size_t MF_LDS_B = (size_t)mf::NT * mf::BSTR;
constexpr size_t MF_LDS_D = (size_t)mf::NT * mf::CB * 4;

// ---------------------------------------------------------------- gate/up

// Workgroup (row tile, work item): rows 64 x .. 64 x + 63 of gate and up for
// the work item's tokens; h = silu(g) * u to LDS, then the Q8_0 of h (two
// 32-row blocks per token) to q_h / d_h of each pair.
template <bool DBG, int WB>
__global__ void __launch_bounds__(256, 3) k_gate_up_mfma(FfnArgs a, const int4 *tiles,
                                                      const int32_t *n_tiles, int8_t *q_h,
                                                      float *d_h) {
  __shared__ __align__(16) uint8_t bs[MF_LDS_B];
  __shared__ float ds[mf::NT * mf::CB];
  __shared__ __align__(16) uint8_t as[2 * mf::RT * mf::astr<WB>()];
  __shared__ __align__(16) float wsl[WB == WB_MX ? 2 * mf::CB * mf::RT : 4];
  __shared__ int tokl[mf::NT], pairl[mf::NT];
  const int rt = blockIdx.x;
  if ((int)blockIdx.y >= *n_tiles) return;
  const int4 t = tiles[blockIdx.y];
  const TileInfo ti = tile_info(a, t);
  const int H = a.H, I = a.I, r0 = rt * mf::RT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid < mf::NT) {
    int tok = 0, pair = 0;
    if (tid < ti.n) tile_tok(a, t, ti.shared, tid, tok, pair);
    tokl[tid] = tok;
    pairl[tid] = pair;
  }
  __syncthreads();
  const size_t row_b = (size_t)H * code_bits<WB>() / 8;
  const uint8_t *mats[2] = {ti.blob, ti.blob + (size_t)I * row_b};
  const uint8_t *tail = ti.blob + 3 * (size_t)I * row_b;  // row scales, or MXFP4 block scales
  const uint8_t *scl[2] = {tail, tail + (size_t)I * (H / 32)};
  float acc[2][4][4];
  int32_t *dots[2] = {a.dbg.gate_dots, a.dbg.up_dots};
  const int m16 = lane & 15, g = lane >> 4;
  // the row scales of this lane's 4 rows, requested with the first chunk
  float sgv[4], suv[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int rl = wv * 16 + g * 4 + i;
    sgv[i] = WB == WB_MX ? 1.0f : gload<float>(tail, 4 * (size_t)(r0 + rl));
    suv[i] = WB == WB_MX ? 1.0f : gload<float>(tail, 4 * ((size_t)I + r0 + rl));
  }
  mfma_kloop_n<2, DBG, WB>(mats, scl, row_b, r0, a.q, a.d, H, tokl, pairl, ti.n, H / 32, bs, ds,
                           as, wsl, acc, dots, I);
  // epilogue: h into LDS as [token][64 rows] fp32 (reuses the activation tile)
  __syncthreads();
  float *hs = reinterpret_cast<float *>(bs);  // 64 x 64 floats = 16 KB <= sizeof(bs)
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int rl = wv * 16 + g * 4 + i;
    const float sg = sgv[i];
    const float su = suv[i];
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const float gv = sg * acc[0][s][i], uv = su * acc[1][s][i];
      const float hv = gv / (1.0f + __expf(-gv)) * uv;
      hs[(s * 16 + m16) * mf::RT + rl] = hv;
      if (DBG && a.dbg.h && s * 16 + m16 < ti.n)
        a.dbg.h[(size_t)pairl[s * 16 + m16] * I + r0 + rl] = hv;
    }
  }
  __syncthreads();
  // Q8_0: 64 tokens x 2 blocks x 8 lanes (4 values each) = 4 passes of 256
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int i = tid + 256 * u, tok_i = i >> 4, blk = (i >> 3) & 1, j = i & 7;
    const float4 v = *reinterpret_cast<const float4 *>(hs + tok_i * mf::RT + blk * 32 + j * 4);
    float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    m = fmaxf(m, __shfl_xor(m, 1, 8));
    m = fmaxf(m, __shfl_xor(m, 2, 8));
    m = fmaxf(m, __shfl_xor(m, 4, 8));
    const float dd = m / 127.0f;
    const float id = dd != 0.0f ? 1.0f / dd : 0.0f;
    auto cv = [&](float f) -> uint32_t {
      const float r = fminf(fmaxf(roundf(f * id), -127.0f), 127.0f);
      return (uint32_t)(uint8_t)(int8_t)(int)r;
    };
    const uint32_t packed = cv(v.x) | (cv(v.y) << 8) | (cv(v.z) << 16) | (cv(v.w) << 24);
    if (tok_i < ti.n) {
      const size_t pair = (size_t)pairl[tok_i];
      reinterpret_cast<uint32_t *>(q_h + pair * I + r0 + blk * 32)[j] = packed;
      if (j == 0) d_h[pair * (I / 32) + (r0 >> 5) + blk] = dd;
      if (DBG && a.dbg.q_h) reinterpret_cast<uint32_t *>(a.dbg.q_h + pair * I + r0 + blk * 32)[j] = packed;
      if (DBG && a.dbg.d_h && j == 0) a.dbg.d_h[pair * (I / 32) + (r0 >> 5) + blk] = dd;
    }
  }
}

// ------------------------------------------------------------------- down

// Workgroup (row tile, work item): output rows 64 x .. of the down matrix
// for the work item's pairs, from Q8_0(h); routed rows go to expert_out of
// the slot, shared rows to shared_out of the token.
template <int TR>
struct DownLds {
  uint8_t bs[TR * mf::BSTR];
  float ds[TR * mf::CB];
  int tokl[TR], pairl[TR];
};

template <bool DBG, int WB, bool NT = false, int TR = mf::NT>
__device__ void down_mfma_tile(const FfnArgs &a, const TileInfo &ti, int rt, const int8_t *q_h,
                               const float *d_h, DownLds<TR> &L, uint8_t *as, float *wsl);

template <bool DBG, int WB>
__global__ void __launch_bounds__(256) k_down_mfma(FfnArgs a, const int4 *tiles,
                                                   const int32_t *n_tiles, const int8_t *q_h,
                                                   const float *d_h) {
  __shared__ __align__(16) DownLds<mf::NT> L;
  __shared__ __align__(16) uint8_t as[mf::RT * mf::astr<WB>()];
  __shared__ __align__(16) float wsl[WB == WB_MX ? mf::CB * mf::RT : 4];
  const int rt = blockIdx.x;
  if ((int)blockIdx.y >= *n_tiles) return;
  const int4 t = tiles[blockIdx.y];
  const TileInfo ti = tile_info(a, t);
  const int tid = threadIdx.x;
  if (tid < mf::NT) {
    int tok = 0, pair = 0;
    if (tid < ti.n) tile_tok(a, t, ti.shared, tid, tok, pair);
    L.tokl[tid] = pair;  // activations of the down projection are indexed by pair
    L.pairl[tid] = pair;
  }
  __syncthreads();
  down_mfma_tile<DBG, WB>(a, ti, rt, q_h, d_h, L, as, wsl);
}

// Down projection of the small-batch layer path for batches of several
// tokens: workgroup (row tile, slot) straight from the batch union's slot
// table (entry: expert, token count, pair ids, record address); empty slots
// exit at once.  A slot holds at most 16 tokens, so 16 activation rows are
// staged per chunk (a quarter of the prefill tiles' LDS and loads).
template <int WB, bool DBG>
__global__ void __launch_bounds__(256) k_down_mfma_slots(FfnArgs a, const int32_t *slots,
                                                         int slot_w, int slot_ptr,
                                                         const int8_t *q_h, const float *d_h) {
  constexpr int TR = 16;
  __shared__ __align__(16) DownLds<TR> L;
  __shared__ __align__(16) uint8_t as[mf::RT * mf::astr<WB>()];
  __shared__ __align__(16) float wsl[WB == WB_MX ? mf::CB * mf::RT : 4];
  const int32_t *ent = slots + (size_t)blockIdx.y * slot_w;
  const int n = ent[1];
  if (n <= 0) return;
  TileInfo ti;
  ti.shared = ent[0] < 0;
  ti.blob = *reinterpret_cast<const uint8_t *const *>(ent + slot_ptr);
  ti.n = min(n, min(a.T, TR));
  const int tid = threadIdx.x;
  const int P = a.T * (a.K + a.n_shared);
  if (tid < TR) {
    const int pair = tid < ti.n ? min(max(ent[2 + tid], 0), P - 1) : 0;
    L.tokl[tid] = pair;
    L.pairl[tid] = pair;
  }
  __syncthreads();
  down_mfma_tile<DBG, WB, true, TR>(a, ti, blockIdx.x, q_h, d_h, L, as, wsl);
}

template <bool DBG, int WB, bool NT, int TR>
__device__ void down_mfma_tile(const FfnArgs &a, const TileInfo &ti, int rt, const int8_t *q_h,
                               const float *d_h, DownLds<TR> &L, uint8_t *as, float *wsl) {
  const int H = a.H, I = a.I, r0 = rt * mf::RT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint8_t *bs = L.bs;
  float *ds = L.ds;
  const int *tokl = L.tokl, *pairl = L.pairl;
  const size_t row_b = (size_t)I * code_bits<WB>() / 8;
  const size_t gate_b = (size_t)I * ((size_t)H * code_bits<WB>() / 8);  // one gate/up matrix
  const uint8_t *mats[1] = {ti.blob + 2 * gate_b};
  const uint8_t *scl[1] = {ti.blob + 3 * gate_b + 2 * (size_t)I * (H / 32)};  // MXFP4
  float acc[1][4][4];
  int32_t *dots[1] = {a.dbg.down_dots};
  mfma_kloop_n<1, DBG, WB, NT, TR>(mats, scl, row_b, r0, q_h, d_h, I, tokl, pairl, ti.n, I / 32, bs,
                               ds, as, wsl, acc, dots, H);
  const int m16 = lane & 15, g = lane >> 4;
  const int row = r0 + wv * 16 + g * 4;  // 4 consecutive rows per lane
  float4 s4 = make_float4(1.0f, 1.0f, 1.0f, 1.0f);  // their row scales
  if constexpr (WB != WB_MX) {
    const uint4 u = gload<uint4>(ti.blob, 3 * gate_b + 4 * ((size_t)2 * I + row));
    s4 = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                     __uint_as_float(u.w));
  }
#pragma unroll
  for (int s = 0; s < TR / 16; s++) {
    const int col = s * 16 + m16;
    if (col >= ti.n) continue;
    const float4 y = make_float4(s4.x * acc[0][s][0], s4.y * acc[0][s][1], s4.z * acc[0][s][2],
                                 s4.w * acc[0][s][3]);
    const int pair = pairl[col];
    float *dst = ti.shared ? a.shared_out + (size_t)(pair - a.T * a.K) * H
                           : a.expert_out + (size_t)pair * H;
    *reinterpret_cast<float4 *>(dst + row) = y;
  }
}

// ------------------------------------------------------------------ launch

size_t mfma_tiles_max(int T, int K, int E, int n_shared) {
  return (size_t)(T * K + mf::NT - 1) / mf::NT + E + (n_shared ? (T + mf::NT - 1) / mf::NT : 0);
}

bool mfma_supported(const FfnArgs &a) {
  return (a.wbits == 4 || a.wbits == 8) && a.H % 256 == 0 && a.I % mf::RT == 0 &&
         a.H % mf::RT == 0 && a.E <= 1024 && a.T > 0;
}

template <bool DBG, int WB>
static void launch_mfma_wb(const FfnArgs &a, int max_tiles, int4 *tiles, int32_t *n_tiles,
                           int8_t *q_h, float *d_h, hipStream_t st, const moe_events *ev) {
  const dim3 g1(a.I / mf::RT, max_tiles), g2(a.H / mf::RT, max_tiles);
  launch_k(k_gate_up_mfma<DBG, WB>, g1, dim3(256), 0, st, stage_ev(ev, MOE_STAGE_GATE_UP), a,
           (const int4 *)tiles, (const int32_t *)n_tiles, q_h, d_h);
  launch_k(k_down_mfma<DBG, WB>, g2, dim3(256), 0, st, stage_ev(ev, MOE_STAGE_DOWN), a,
           (const int4 *)tiles, (const int32_t *)n_tiles, (const int8_t *)q_h,
           (const float *)d_h);
}

template <bool DBG>
static void launch_down_slots_dbg(const FfnArgs &a, const int32_t *slots, int n_slots_ub,
                                  int slot_w, int slot_ptr, const int8_t *q_h, const float *d_h,
                                  hipStream_t st, const moe_events *ev) {
  const dim3 g(a.H / mf::RT, n_slots_ub);
  const Ev ed = stage_ev(ev, MOE_STAGE_DOWN);
  if (a.wfmt == 1)
    launch_k(k_down_mfma_slots<WB_MX, DBG>, g, dim3(256), 0, st, ed, a, slots, slot_w, slot_ptr,
             q_h, d_h);
  else if (a.wbits == 8)
    launch_k(k_down_mfma_slots<8, DBG>, g, dim3(256), 0, st, ed, a, slots, slot_w, slot_ptr, q_h,
             d_h);
  else if (a.wbits == 2)
    launch_k(k_down_mfma_slots<2, DBG>, g, dim3(256), 0, st, ed, a, slots, slot_w, slot_ptr, q_h,
             d_h);
  else
    launch_k(k_down_mfma_slots<4, DBG>, g, dim3(256), 0, st, ed, a, slots, slot_w, slot_ptr, q_h,
             d_h);
}

void launch_down_mfma_slots(const FfnArgs &a, const int32_t *slots, int n_slots_ub, int slot_w,
                            int slot_ptr, const int8_t *q_h, const float *d_h, bool dbg,
                            hipStream_t st, const moe_events *ev) {
  if (dbg) launch_down_slots_dbg<true>(a, slots, n_slots_ub, slot_w, slot_ptr, q_h, d_h, st, ev);
  else launch_down_slots_dbg<false>(a, slots, n_slots_ub, slot_w, slot_ptr, q_h, d_h, st, ev);
}

void launch_mfma_tiles(const FfnArgs &a, int4 *tiles, int32_t *n_tiles, hipStream_t st) {
  hipLaunchKernelGGL(k_mfma_tiles, dim3(1), dim3(256), 0, st, a.E, a.T, a.n_shared, a.offsets,
                     tiles, n_tiles);
}

void launch_ffn_mfma(const FfnArgs &a, int4 *tiles, int32_t *n_tiles, int8_t *q_h, float *d_h,
                     hipStream_t st, const moe_events *ev) {
  const int max_tiles = (int)mfma_tiles_max(a.T, a.K, a.E, a.n_shared);
  launch_mfma_tiles(a, tiles, n_tiles, st);
  const bool dbg = a.dbg.gate_dots || a.dbg.up_dots || a.dbg.h || a.dbg.q_h || a.dbg.d_h ||
                   a.dbg.down_dots;
  if (a.wfmt == 1) {
    if (dbg) launch_mfma_wb<true, WB_MX>(a, max_tiles, tiles, n_tiles, q_h, d_h, st, ev);
    else launch_mfma_wb<false, WB_MX>(a, max_tiles, tiles, n_tiles, q_h, d_h, st, ev);
  } else if (a.wbits == 8) {
    if (dbg) launch_mfma_wb<true, 8>(a, max_tiles, tiles, n_tiles, q_h, d_h, st, ev);
    else launch_mfma_wb<false, 8>(a, max_tiles, tiles, n_tiles, q_h, d_h, st, ev);
  } else {
    if (dbg) launch_mfma_wb<true, 4>(a, max_tiles, tiles, n_tiles, q_h, d_h, st, ev);
    else launch_mfma_wb<false, 4>(a, max_tiles, tiles, n_tiles, q_h, d_h, st, ev);
  }
}

}  // namespace moe

// Expert FFNs with per-row activation scales (moe_cfg.act_block =
// MOE_ACT_ROW): grouped int4/int8 x int8 GEMMs on the matrix cores with one
// integer accumulator per output row.
//
// The format ("Show HN: 遅いコンピュータで GLM 5.2 を実行する", section
// 実装済みの主な機能, integer-dot item, with the activation scale taken per row
// instead of per 32 values): x has one fp32 scale per token row, h one per
// (token, expert) row, so
//   g[t,r] = sg[r] * (d[t] * P),   P = sum over the whole row of code * q
// exactly in int32 (|P| <= 16 * 6144 * 8 * 127 < 2^31, int4 codes entering as
// 16 x code).  With no per-block scaling the contraction runs on the K = 64
// int8 MFMA of gfx950 (v_mfma_i32_16x16x64_i8, twice the work per
// instruction of the K = 32 one) with no fix-up arithmetic in the inner loop.
//
// A workgroup computes 4 x 16 RS rows x 64 tokens of one work item (expert,
// token tile), 4 waves of 16 RS rows, gate and up together in the gate/up
// kernel; RS = 2 (32 rows per wave): with RS = 1 three workgroups fit on a
// CU instead of two, but every MFMA then needs twice the activation bytes
// from LDS, and both GEMMs ran slower (dense 2048-token int4 gate/up 0.349
// against 0.369 of the int8 peak, down 0.245 against 0.280).  K
// runs in chunks staged in LDS (weights as packed codes, activations
// reordered like the nibble split for int4), the next chunk in registers
// meanwhile.  Row strides in LDS are padded so that the 8-byte (int4
// weights) and 16-byte (int8 weights, activations) fragment reads of a wave
// hit distinct banks.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {

// row sub-tiles of 16 per wave (2: 32 rows per wave, 128 per workgroup)
#ifndef MOE_ROWS_RS
#define MOE_ROWS_RS 2
#endif

namespace mr {
constexpr int NT = TILE_T;       // tokens per work item
constexpr int RS = MOE_ROWS_RS;  // 16-row sub-tiles per wave
constexpr int RW = 16 * RS;      // rows per wave
constexpr int RT = 4 * RW;       // rows per workgroup
template <int WB>
constexpr int KC() { return WB == 8 ? 128 : 256; }  // K (codes) per chunk: 128 bytes of a row
template <int WB>
constexpr int ASTR() { return WB == 8 ? 128 + 16 : 128 + 8; }  // LDS bytes per weight row
template <int WB>
constexpr int BSTR() { return KC<WB>() + 16; }  // LDS bytes per activation row
}  // namespace mr

// One K chunk in registers: NM weight matrices x RT rows x 128 bytes, and
// 64 activation rows x KC bytes, as 16-byte pieces per thread.
template <int NM, int WB>
struct RChunk {
  static constexpr int AP = NM * mr::RT * 8 / 256;          // weight pieces per thread
  static constexpr int BPR = mr::KC<WB>() / 16;             // pieces per activation row
  static constexpr int BP = mr::NT * BPR / 256;             // activation pieces per thread
  uint4 a[AP];
  uint4 b[BP];
};

// Chunk c: rows r0.. of each matrix (row_b bytes of codes per row) and the
// activation rows tokl[] (row_len int8 each).  Every load is unconditional:
// a piece past the end of a row reads the row's last 16 bytes (the step
// loop stops at the row's end, so those are never used).
template <int NM, int WB>
__device__ __forceinline__ void rload(const uint8_t *const *mat, size_t row_b, int r0,
                                      const int8_t *q, int row_len, const int *tokl, int c,
                                      RChunk<NM, WB> &r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < RChunk<NM, WB>::AP; u++) {
    const int i = tid + 256 * u, m = i / (mr::RT * 8), rem = i % (mr::RT * 8);
    const int row = rem / 8, pc = rem % 8;
    size_t off = (size_t)c * 128 + pc * 16;
    off = off + 16 <= row_b ? off : row_b - 16;
    r.a[u] = gload<uint4>(mat[m], (size_t)(r0 + row) * row_b + off);
  }
  constexpr int BPR = RChunk<NM, WB>::BPR;
#pragma unroll
  for (int u = 0; u < RChunk<NM, WB>::BP; u++) {
    const int i = tid + 256 * u, tok = i / BPR, pc = i % BPR;
    int off = c * mr::KC<WB>() + pc * 16;
    off = off + 16 <= row_len ? off : row_len - 16;
    r.b[u] = gload<uint4>(reinterpret_cast<const uint8_t *>(q),
                          (size_t)tokl[tok] * row_len + off);
  }
}

template <int NM, int WB>
__device__ __forceinline__ void rstore(const RChunk<NM, WB> &r, uint8_t *as, uint8_t *bs) {
  const int tid = threadIdx.x;
  constexpr int AS = mr::ASTR<WB>(), BS = mr::BSTR<WB>();
#pragma unroll
  for (int u = 0; u < RChunk<NM, WB>::AP; u++) {
    const int i = tid + 256 * u, m = i / (mr::RT * 8), rem = i % (mr::RT * 8);
    uint8_t *dst = as + (size_t)(m * mr::RT + rem / 8) * AS + (rem % 8) * 16;
    if constexpr (WB == 8) {  // rows 16-byte aligned
      *reinterpret_cast<uint4 *>(dst) = r.a[u];
    } else {  // rows 8-byte aligned
      reinterpret_cast<uint2 *>(dst)[0] = make_uint2(r.a[u].x, r.a[u].y);
      reinterpret_cast<uint2 *>(dst)[1] = make_uint2(r.a[u].z, r.a[u].w);
    }
  }
  constexpr int BPR = RChunk<NM, WB>::BPR;
#pragma unroll
  for (int u = 0; u < RChunk<NM, WB>::BP; u++) {
    const int i = tid + 256 * u;
    uint4 v = r.b[u];
    if constexpr (WB != 8) {  // even codes, then odd, per 8 (the nibble split)
      const uint2 e0 = even_odd8(v.x, v.y), e1 = even_odd8(v.z, v.w);
      v = make_uint4(e0.x, e0.y, e1.x, e1.y);
    }
    *reinterpret_cast<uint4 *>(bs + (size_t)(i / BPR) * BS + (i % BPR) * 16) = v;
  }
}

// The K loop: acc[m][rs][s] = 16x16 int32 tile of matrix m, rows 16 rs of
// the wave's 32, tokens 16 s (NS sub-tiles hold tokens), over the K codes of
// the rows.  Lane (n = lane % 16, g = lane / 16) feeds codes and activations
// 16 g .. 16 g + 15 of each 64-step to the MFMA (for int4: 8 packed bytes
// unpacked to 16 x code, even codes first, matching the staged activations).
template <int NM, int NS, int WB>
__device__ void rkloop(const uint8_t *const *mat, size_t row_b, int r0, const int8_t *q,
                       const int *tokl, int K, uint8_t *as, uint8_t *bs,
                       v4i (&acc)[NM][mr::RS][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m16 = lane & 15, g = lane >> 4;
  constexpr int KC = mr::KC<WB>(), AS = mr::ASTR<WB>(), BS = mr::BSTR<WB>();
#pragma unroll
  for (int m = 0; m < NM; m++)
#pragma unroll
    for (int rs = 0; rs < mr::RS; rs++)
#pragma unroll
      for (int s = 0; s < 4; s++) acc[m][rs][s] = v4i{0, 0, 0, 0};
  const int nchunk = (K + KC - 1) / KC;
  RChunk<NM, WB> rc;
  rload<NM, WB>(mat, row_b, r0, q, K, tokl, 0, rc);
  for (int c = 0; c < nchunk; c++) {
    __syncthreads();  // the previous chunk is consumed
    rstore<NM, WB>(rc, as, bs);
    __syncthreads();
    if (c + 1 < nchunk) rload<NM, WB>(mat, row_b, r0, q, K, tokl, c + 1, rc);
    const int steps = min(KC, K - c * KC) / 64;
#pragma unroll
    for (int st = 0; st < KC / 64; st++) {
      if (st < steps) {
        v4i af[NM][mr::RS];
#pragma unroll
        for (int m = 0; m < NM; m++)
#pragma unroll
          for (int rs = 0; rs < mr::RS; rs++) {
            const uint8_t *ar = as + (size_t)(m * mr::RT + wv * mr::RW + rs * 16 + m16) * AS;
            if constexpr (WB == 8) {
              const uint4 w = *reinterpret_cast<const uint4 *>(ar + st * 64 + g * 16);
              af[m][rs] = v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
            } else {
              const uint2 w = *reinterpret_cast<const uint2 *>(ar + st * 32 + g * 8);
              af[m][rs] = v4i{lo16(w.x), hi16(w.x), lo16(w.y), hi16(w.y)};
            }
          }
#pragma unroll
        for (int s = 0; s < NS; s++) {
          const uint4 b = *reinterpret_cast<const uint4 *>(bs + (size_t)(s * 16 + m16) * BS +
                                                           st * 64 + g * 16);
          const v4i bf = {(int)b.x, (int)b.y, (int)b.z, (int)b.w};
#pragma unroll
          for (int m = 0; m < NM; m++)
#pragma unroll
            for (int rs = 0; rs < mr::RS; rs++)
              acc[m][rs][s] =
                  __builtin_amdgcn_mfma_i32_16x16x64_i8(af[m][rs], bf, acc[m][rs][s], 0, 0, 0);
        }
      }
    }
  }
}

template <int NM, int WB>
__device__ void rkloop_n(const uint8_t *const *mat, size_t row_b, int r0, const int8_t *q,
                         const int *tokl, int K, int n, uint8_t *as, uint8_t *bs,
                         v4i (&acc)[NM][mr::RS][4]) {
  switch ((n + 15) / 16) {
    case 1: rkloop<NM, 1, WB>(mat, row_b, r0, q, tokl, K, as, bs, acc); break;
    case 2: rkloop<NM, 2, WB>(mat, row_b, r0, q, tokl, K, as, bs, acc); break;
    case 3: rkloop<NM, 3, WB>(mat, row_b, r0, q, tokl, K, as, bs, acc); break;
    default: rkloop<NM, 4, WB>(mat, row_b, r0, q, tokl, K, as, bs, acc);
  }
}

// Workgroup (row tile, work item): rows RT x .. of gate and up for the work
// item's tokens; h = silu(g) * u (fp32) to hbuf [P][I], quantised per row by
// the next kernel once every row tile of the pair is written.
template <bool DBG, int WB>
__global__ void __launch_bounds__(256) k_gate_up_rows(FfnArgs a, const int4 *tiles,
                                                      const int32_t *n_tiles, float *hbuf) {
  __shared__ __align__(16) uint8_t as[2 * mr::RT * mr::ASTR<WB>()];
  __shared__ __align__(16) uint8_t bs[mr::NT * mr::BSTR<WB>()];
  __shared__ int tokl[mr::NT], pairl[mr::NT];
  __shared__ float dtok[mr::NT];
  const int rt = blockIdx.x;
  if ((int)blockIdx.y >= *n_tiles) return;
  const int4 t = tiles[blockIdx.y];
  const TileInfo ti = tile_info(a, t);
  const int H = a.H, I = a.I, r0 = rt * mr::RT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m16 = lane & 15, g = lane >> 4;
  if (tid < mr::NT) {
    int tok = 0, pair = 0;
    if (tid < ti.n) tile_tok(a, t, ti.shared, tid, tok, pair);
    tokl[tid] = tok;
    pairl[tid] = pair;
    // the token's row scale; int4 codes enter the MFMA as 16 x code
    dtok[tid] = a.d[tok] * (WB == 8 ? 1.0f : 0.0625f);
  }
  __syncthreads();
  const size_t row_b = (size_t)H * code_bits<WB>() / 8;
  const uint8_t *mats[2] = {ti.blob, ti.blob + (size_t)I * row_b};
  const uint8_t *tail = ti.blob + 3 * (size_t)I * row_b;
  float4 sc[2][mr::RS];  // row scales of this lane's 4 rows: [gate, up][rs]
#pragma unroll
  for (int m = 0; m < 2; m++)
#pragma unroll
    for (int rs = 0; rs < mr::RS; rs++) {
      const uint4 u = gload<uint4>(tail, 4 * ((size_t)m * I + r0 + wv * mr::RW + rs * 16 + g * 4));
      sc[m][rs] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                              __uint_as_float(u.w));
    }
  v4i acc[2][mr::RS][4];
  rkloop_n<2, WB>(mats, row_b, r0, a.q, tokl, H, ti.n, as, bs, acc);
#pragma unroll
  for (int rs = 0; rs < mr::RS; rs++) {
    const int row = r0 + wv * mr::RW + rs * 16 + g * 4;  // 4 consecutive rows per lane
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const int col = s * 16 + m16;
      if (col >= ti.n) continue;
      const float dt = dtok[col];
      const size_t pair = (size_t)pairl[col];
      const float sg[4] = {sc[0][rs].x, sc[0][rs].y, sc[0][rs].z, sc[0][rs].w};
      const float su[4] = {sc[1][rs].x, sc[1][rs].y, sc[1][rs].z, sc[1][rs].w};
      float hv[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float gv = sg[i] * (dt * (float)acc[0][rs][s][i]);
        const float uv = su[i] * (dt * (float)acc[1][rs][s][i]);
        hv[i] = gv / (1.0f + __expf(-gv)) * uv;
      }
      *reinterpret_cast<float4 *>(hbuf + pair * I + row) = make_float4(hv[0], hv[1], hv[2], hv[3]);
      if constexpr (DBG) {  // one int32 dot per row: dumps [P][I][1]
#pragma unroll
        for (int i = 0; i < 4; i++) {
          if (a.dbg.gate_dots) a.dbg.gate_dots[pair * I + row + i] = acc[0][rs][s][i] >> (WB == 8 ? 0 : 4);
          if (a.dbg.up_dots) a.dbg.up_dots[pair * I + row + i] = acc[1][rs][s][i] >> (WB == 8 ? 0 : 4);
          if (a.dbg.h) a.dbg.h[pair * I + row + i] = hv[i];
        }
      }
    }
  }
}

// Workgroup (row tile, work item): output rows RT x .. of the down matrix
// for the work item's pairs, from their per-row quantised h; routed rows to
// expert_out of the slot, shared rows to shared_out of the token.
template <bool DBG, int WB>
__global__ void __launch_bounds__(256) k_down_rows(FfnArgs a, const int4 *tiles,
                                                   const int32_t *n_tiles, const int8_t *q_h,
                                                   const float *d_h) {
  __shared__ __align__(16) uint8_t as[mr::RT * mr::ASTR<WB>()];
  __shared__ __align__(16) uint8_t bs[mr::NT * mr::BSTR<WB>()];
  __shared__ int pairl[mr::NT];
  __shared__ float dtok[mr::NT];
  const int rt = blockIdx.x;
  if ((int)blockIdx.y >= *n_tiles) return;
  const int4 t = tiles[blockIdx.y];
  const TileInfo ti = tile_info(a, t);
  const int H = a.H, I = a.I, r0 = rt * mr::RT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m16 = lane & 15, g = lane >> 4;
  if (tid < mr::NT) {
    int tok = 0, pair = 0;
    if (tid < ti.n) tile_tok(a, t, ti.shared, tid, tok, pair);
    pairl[tid] = pair;  // the down projection's activations are indexed by pair
    dtok[tid] = d_h[pair] * (WB == 8 ? 1.0f : 0.0625f);
  }
  __syncthreads();
  const size_t row_b = (size_t)I * code_bits<WB>() / 8;
  const size_t gate_b = (size_t)I * ((size_t)H * code_bits<WB>() / 8);  // one gate/up matrix
  const uint8_t *mats[1] = {ti.blob + 2 * gate_b};
  float4 sd[mr::RS];
#pragma unroll
  for (int rs = 0; rs < mr::RS; rs++) {
    const uint4 u =
        gload<uint4>(ti.blob, 3 * gate_b + 4 * ((size_t)2 * I + r0 + wv * mr::RW + rs * 16 + g * 4));
    sd[rs] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                         __uint_as_float(u.w));
  }
  v4i acc[1][mr::RS][4];
  rkloop_n<1, WB>(mats, row_b, r0, q_h, pairl, I, ti.n, as, bs, acc);
#pragma unroll
  for (int rs = 0; rs < mr::RS; rs++) {
    const int row = r0 + wv * mr::RW + rs * 16 + g * 4;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const int col = s * 16 + m16;
      if (col >= ti.n) continue;
      const float dt = dtok[col];
      const int pair = pairl[col];
      const float4 y = make_float4(sd[rs].x * (dt * (float)acc[0][rs][s][0]),
                                   sd[rs].y * (dt * (float)acc[0][rs][s][1]),
                                   sd[rs].z * (dt * (float)acc[0][rs][s][2]),
                                   sd[rs].w * (dt * (float)acc[0][rs][s][3]));
      float *dst = ti.shared ? a.shared_out + (size_t)(pair - a.T * a.K) * H
                             : a.expert_out + (size_t)pair * H;
      *reinterpret_cast<float4 *>(dst + row) = y;
      if constexpr (DBG) {
        if (a.dbg.down_dots) {
#pragma unroll
          for (int i = 0; i < 4; i++)
            a.dbg.down_dots[(size_t)pair * H + row + i] = acc[0][rs][s][i] >> (WB == 8 ? 0 : 4);
        }
      }
    }
  }
}

bool mfma_rows_supported(const FfnArgs &a) {
  return (a.wbits == 4 || a.wbits == 8) && a.wfmt == 0 && a.H % mr::RT == 0 &&
         a.I % mr::RT == 0 && a.H % 64 == 0 && a.I % 64 == 0 && a.E <= 1024 && a.T > 0;
}

template <bool DBG, int WB>
static void launch_rows_wb(const FfnArgs &a, int max_tiles, int4 *tiles, int32_t *n_tiles,
                           float *h, int8_t *q_h, float *d_h, const int32_t *idx,
                           hipStream_t st, const moe_events *ev) {
  const dim3 g1(a.I / mr::RT, max_tiles), g2(a.H / mr::RT, max_tiles);
  launch_k(k_gate_up_rows<DBG, WB>, g1, dim3(256), 0, st, stage_ev(ev, MOE_STAGE_GATE_UP), a,
           (const int4 *)tiles, (const int32_t *)n_tiles, h);
  const int P = a.T * a.K + a.T * a.n_shared;
  launch_quant_rows(h, q_h, d_h, P, a.I, idx, a.T * a.K, st);
  launch_k(k_down_rows<DBG, WB>, g2, dim3(256), 0, st, stage_ev(ev, MOE_STAGE_DOWN), a,
           (const int4 *)tiles, (const int32_t *)n_tiles, (const int8_t *)q_h, (const float *)d_h);
}

void launch_ffn_mfma_rows(const FfnArgs &a, int4 *tiles, int32_t *n_tiles, float *h, int8_t *q_h,
                          float *d_h, const int32_t *idx, hipStream_t st, const moe_events *ev) {
  const int max_tiles = (int)mfma_tiles_max(a.T, a.K, a.E, a.n_shared);
  launch_mfma_tiles(a, tiles, n_tiles, st);
  const bool dbg = a.dbg.gate_dots || a.dbg.up_dots || a.dbg.h || a.dbg.down_dots;
  if (a.wbits == 8) {
    if (dbg) launch_rows_wb<true, 8>(a, max_tiles, tiles, n_tiles, h, q_h, d_h, idx, st, ev);
    else launch_rows_wb<false, 8>(a, max_tiles, tiles, n_tiles, h, q_h, d_h, idx, st, ev);
  } else {
    if (dbg) launch_rows_wb<true, 4>(a, max_tiles, tiles, n_tiles, h, q_h, d_h, idx, st, ev);
    else launch_rows_wb<false, 4>(a, max_tiles, tiles, n_tiles, h, q_h, d_h, idx, st, ev);
  }
}

}  // namespace moe

// Internal launch entry points of the libmoe kernels (host side).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Sets the calling thread's message for moe_last_error and returns code.
int set_error(int code, const char *msg);

// Kernel timestamps: a stage launched with a non-null event pair goes through
// hipExtLaunchKernelGGL, which stamps the events from the kernel's own
// dispatch (no extra queue packets).
struct Ev {
  hipEvent_t start = nullptr, stop = nullptr;
};
inline Ev stage_ev(const moe_events *e, int stage) {
  Ev r;
  if (e) {
    r.start = (hipEvent_t)e->start[stage];
    r.stop = (hipEvent_t)e->stop[stage];
  }
  return r;
}
template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 g, dim3 b, uint32_t lds, hipStream_t st, Ev ev, Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, g, b, lds, st, ev.start, ev.stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, g, b, lds, st, args...);
}

void launch_quant_act(const float *x, int8_t *q, float *d, int64_t n_elems, hipStream_t st,
                      const moe_events *ev = nullptr);
// The per-row activation format: one scale per row of n floats (rows r <
// n_skip with skip[r] < 0 are not written; skip may be NULL).
void launch_quant_rows(const float *x, int8_t *q, float *d, int64_t rows, int n,
                       const int32_t *skip, int n_skip, hipStream_t st,
                       const moe_events *ev = nullptr);
void launch_combine(int T, int H, int K, const float *eo, const float *w, const float *shared,
                    const float *residual, float *y, float *yn, float eps, hipStream_t st,
                    const moe_events *ev = nullptr);
void launch_rmsnorm(int T, int H, const float *x, float *y, float eps, hipStream_t st);

// Router: scores into s/sb [T][E] (workspace, route.hip), then selection
// into idx/w (one workgroup per token, decode.hip).
void launch_router_scores(const moe_cfg &c, int T, const float *x, const float *wr,
                          const float *bias, float *s, float *sb, hipStream_t st,
                          const moe_events *ev = nullptr);
void launch_router_select(const moe_cfg &c, int T, const float *s, const float *sb,
                          int32_t *idx, float *w, hipStream_t st, const moe_events *ev = nullptr);

void launch_group(int n_slots, int E, const int32_t *idx, int32_t *counts, int32_t *offsets,
                  int32_t *perm, int32_t *inv, int32_t *active, int32_t *n_active,
                  hipStream_t st, const moe_events *ev = nullptr);

// Expert FFN over grouped tokens (dot-product GEMV path).
struct FfnArgs {
  int H, I, E, K, T, n_shared, wbits;
  int wfmt;  // 0: integer codes with row scales; 1: MXFP4; 2: FP8 with 128x128 block scales
  size_t blob_bytes;
  const int8_t *q;
  const float *d;
  const uint8_t *experts;
  const uint8_t *const *expert_ptrs;  // nullable: per-expert record pointers
  const uint8_t *shared;
  const int32_t *offsets, *perm, *active, *n_active;
  float *h;        // [P][I] fp32 workspace
  float *expert_out;
  float *shared_out;
  moe_ffn_debug dbg;
};
void launch_ffn_gemv(const FfnArgs &a, hipStream_t st, const moe_events *ev = nullptr);
// FP8 E4M3 experts with 128x128 block scales (wfmt 2), every batch size:
// vector gate/up and down with exact int32 block dots (ffn_gemv.hip).
bool f8_supported(const FfnArgs &a);
void launch_ffn_f8(const FfnArgs &a, hipStream_t st, const moe_events *ev = nullptr);

// Expert FFN over grouped tokens on the matrix cores (ffn_mfma.hip): tile list
// from the grouping offsets, then grouped gate/up (Q8_0 of h into q_h/d_h,
// [P][I] and [P][I/32]) and grouped down into expert_out / shared_out.
size_t mfma_tiles_max(int T, int K, int E, int n_shared);
bool mfma_supported(const FfnArgs &a);
// The tile list alone (one workgroup): work items (expert, first list
// position, token count) of TILE_T tokens from the grouping offsets.
void launch_mfma_tiles(const FfnArgs &a, int4 *tiles, int32_t *n_tiles, hipStream_t st);
void launch_ffn_mfma(const FfnArgs &a, int4 *tiles, int32_t *n_tiles, int8_t *q_h, float *d_h,
                     hipStream_t st, const moe_events *ev = nullptr);
// The same with one activation scale per row (the per-row format): q, d of
// x per token row; gate/up writes fp32 h [P][I], which is quantised per
// (token, expert) row into q_h [P][I] / d_h [P] (pairs of slots dropped by
// top-p, idx[p] < 0, skipped), then the down projection.  Int4 and int8
// codes.  Dumps: one int32 dot per row ([P][I][1], [P][H][1]) and h.
bool mfma_rows_supported(const FfnArgs &a);
void launch_ffn_mfma_rows(const FfnArgs &a, int4 *tiles, int32_t *n_tiles, float *h, int8_t *q_h,
                          float *d_h, const int32_t *idx, hipStream_t st,
                          const moe_events *ev = nullptr);
// The down projection of the small-batch path from its slot table (int8,
// int4, MXFP4), rows to expert_out / shared_out.
// dbg: the kernel that also writes a.dbg.down_dots.
void launch_down_mfma_slots(const FfnArgs &a, const int32_t *slots, int n_slots_ub, int slot_w,
                            int slot_ptr, const int8_t *q_h, const float *d_h, bool dbg,
                            hipStream_t st, const moe_events *ev);

// Whole layer for 1..16 tokens in four kernels (decode.h).
struct LayerArgs {
  int H, I, E, G, TG, K, T, n_shared, wbits;
  int wfmt;  // 0: integer codes with row scales; 1: MXFP4; 2: FP8 with 128x128 block scales
  float scale, eps;
  float top_p;  // adaptive expert top-p; 0 or 1 = off
  size_t blob_bytes;
  const float *x, *wr, *bias, *residual;
  const uint8_t *experts, *shared;
  const uint8_t *const *expert_ptrs;  // nullable: per-expert record pointers
  float *y, *y_norm;
  int32_t *idx;
  float *w;
  float *s, *sb;                 // [T][E] router scores
  int8_t *q;                     // [T][H] Q8_0 of x
  float *d;                      // [T][H/32]
  int32_t *slots;                // [n_slots_ub][2 + 2*16] slot table
  float *hs;                     // [T][I] shared expert's h (fp32)
  int8_t *qh;                    // [P][I] Q8_0 of h
  float *dh;                     // [P][I/32]
  float *ssq;                    // [T][H/8] partial sums of squares
  float *eo_r, *eo_s;            // expert_out [T*K][H] / shared_out [T][H] (MFMA down)
  int n_slots_ub;
  moe_layer_debug dbg;           // dumps (launch_small_batch_dbg only)
};
size_t small_batch_slot_ints(int T, int K, int n_shared);
// Matrix cores alone (peak.hip): n_wg workgroups of 4 waves, each wave
// iters x 8 int8 MFMAs (16x16x64); out [n_wg * 256] takes a checksum.
void launch_mfma_peak(int n_wg, int iters, int32_t *out, hipStream_t st);
// A plain streaming read of bytes (a multiple of 16) for the HBM read rate
// (peak.hip); one checksum word per wave into out [n_wg * 4]; ev: optional
// timestamps of the kernel's own dispatch.
void launch_read_peak(const void *buf, int64_t bytes, int n_wg, uint32_t *out, hipStream_t st,
                      Ev ev);

bool small_batch_supported(const moe_cfg &c, int T);
void launch_small_batch(LayerArgs a, hipStream_t st, const moe_events *ev);
// The same with a.dbg's dumps written (decode_dbg.hip).
void launch_small_batch_dbg(LayerArgs a, hipStream_t st, const moe_events *ev);

}  // namespace moe

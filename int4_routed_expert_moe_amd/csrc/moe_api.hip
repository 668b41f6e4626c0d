// libmoe C ABI: argument validation, workspace layout and kernel launches.
// Every entry point either enqueues all of its work on the given stream and
// returns MOE_OK, or returns an error code having enqueued nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kernels.h"

namespace {

thread_local char g_msg[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace

namespace moe {
int set_error(int code, const char *msg) {
  snprintf(g_msg, sizeof(g_msg), "%s", msg);
  return code;
}
}  // namespace moe

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

// smallest batch whose expert FFNs run as grouped MFMA GEMMs (int4 / int2)
#ifndef MOE_MFMA_MIN_T
#define MOE_MFMA_MIN_T 17
#endif

int check_cfg(const moe_cfg *c) {
  if (!c) return fail(MOE_EINVAL, "cfg is NULL");
  if (c->hidden <= 0 || c->hidden % 256)
    return fail(MOE_EINVAL, "hidden=%d must be a positive multiple of 256", c->hidden);
  if (c->inter <= 0 || c->inter % 128)
    return fail(MOE_EINVAL, "inter=%d must be a positive multiple of 128", c->inter);
  if (c->wbits != 8 && c->wbits != 4 && c->wbits != 2)
    return fail(MOE_EINVAL, "wbits=%d not in {8,4,2}", c->wbits);
  const int per = 128 / c->wbits;  // codes per 16-byte piece
  if (c->hidden / per > (c->wbits == 8 ? 448 : 256) || c->inter / per > 128)
    return fail(MOE_EINVAL, "hidden=%d / inter=%d too large for wbits=%d", c->hidden, c->inter,
                c->wbits);
  if (c->n_experts < 2 || c->n_experts > 1024)
    return fail(MOE_EINVAL, "n_experts=%d not in [2,1024]", c->n_experts);
  if (c->n_group < 1 || c->n_group > 64 || c->n_experts % c->n_group ||
      c->n_experts / c->n_group < 2)
    return fail(MOE_EINVAL, "n_group=%d must divide n_experts=%d into groups of >= 2 (<= 64 groups)",
                c->n_group, c->n_experts);
  if (c->topk_group < 1 || c->topk_group > c->n_group)
    return fail(MOE_EINVAL, "topk_group=%d not in [1, n_group]", c->topk_group);
  const int cand = c->topk_group * (c->n_experts / c->n_group);
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > cand)
    return fail(MOE_EINVAL, "top_k=%d not in [1, min(16, %d)]", c->top_k, cand);
  if (c->n_shared != 0 && c->n_shared != 1)
    return fail(MOE_EINVAL, "n_shared=%d not in {0,1}", c->n_shared);
  if (!(c->routed_scaling > 0.0f) || c->routed_scaling > 1e30f)
    return fail(MOE_EINVAL, "routed_scaling must be finite and > 0");
  if (!(c->top_p >= 0.0f && c->top_p <= 1.0f))
    return fail(MOE_EINVAL, "top_p must be 0 (off) or in (0, 1]");
  if (c->wfmt < 0 || c->wfmt > 2) return fail(MOE_EINVAL, "wfmt=%d not in {0,1,2}", c->wfmt);
  if (c->wfmt == 1 && c->wbits != 4)
    return fail(MOE_EINVAL, "MXFP4 experts (wfmt 1) need wbits 4 (4-bit codes)");
  if (c->wfmt == 2 && c->wbits != 8)
    return fail(MOE_EINVAL, "FP8 experts (wfmt 2) need wbits 8 (byte codes)");
  if (c->act_block != 0 && c->act_block != 32 && c->act_block != MOE_ACT_ROW)
    return fail(MOE_EINVAL, "act_block=%d not in {0, 32, MOE_ACT_ROW}", c->act_block);
  if (c->act_block == MOE_ACT_ROW && (c->wfmt != 0 || (c->wbits != 4 && c->wbits != 8)))
    return fail(MOE_EINVAL, "per-row activation scales need int4 or int8 codes (wfmt 0)");
  return MOE_OK;
}

bool act_rows(const moe_cfg &c) { return c.act_block == MOE_ACT_ROW; }

// Byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return a && b && x < y + nb && y < x + na;
}

#define REQUIRE(p, name)                                                       \
  do {                                                                         \
    if (!(p)) return fail(MOE_EINVAL, "%s is NULL", name);                     \
    if (!aligned((p), 16)) return fail(MOE_EALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

#define OPTIONAL(p, name)                                                      \
  do {                                                                         \
    if ((p) && !aligned((p), 16)) return fail(MOE_EALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

// HIP's per-thread last-error state is cleared on entry to every call that
// launches work, so that launched() sees only this call's own launches (an
// earlier failed HIP call of the caller would otherwise be reported here).
void clear_hip_error() { (void)hipGetLastError(); }

int launched(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

size_t blob_bytes(const moe_cfg &c) {
  const size_t elems = (size_t)2 * c.inter * c.hidden + (size_t)c.hidden * c.inter;
  if (c.wfmt == 1) return elems / 2 + elems / 32;  // FP4 codes + one E8M0 byte per 32
  if (c.wfmt == 2)  // E4M3 bytes + one fp32 scale per 128x128 block of each matrix
    return elems + sizeof(float) * 3 * (size_t)(c.inter / 128) * (c.hidden / 128);
  return elems * (size_t)c.wbits / 8 + sizeof(float) * ((size_t)2 * c.inter + c.hidden);
}

// workspace carving --------------------------------------------------------
struct Carve {
  uint8_t *base;
  size_t off = 0;
  template <class T>
  T *take(size_t n) {
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += up256(n * sizeof(T));
    return p;
  }
};

struct RouteWs {
  float *s, *sb;
};
RouteWs carve_route(Carve &cv, const moe_cfg &c, int T) {
  RouteWs r;
  r.s = cv.take<float>((size_t)T * c.n_experts);
  r.sb = cv.take<float>((size_t)T * c.n_experts);
  return r;
}

struct FfnWs {
  int32_t *counts, *offsets, *perm, *inv, *active, *n_active;
  int32_t *n_tiles;
  int4 *tiles;
  float *h;  // fp32 h [P][I] (GEMV path); the MFMA path keeps Q8_0(h) here
  int8_t *qh_rows;  // per-row activations: q_h [P][I] and d_h [P] (h stays fp32)
  float *dh_rows;
};
FfnWs carve_ffn(Carve &cv, const moe_cfg &c, int T) {
  FfnWs f;
  const size_t slots = (size_t)T * c.top_k;
  const size_t pairs = slots + (size_t)T * c.n_shared;
  f.counts = cv.take<int32_t>(c.n_experts);
  f.offsets = cv.take<int32_t>(c.n_experts + 1);
  f.perm = cv.take<int32_t>(slots);
  f.inv = cv.take<int32_t>(slots);
  f.active = cv.take<int32_t>(c.n_experts);
  f.n_active = cv.take<int32_t>(1);
  f.n_tiles = cv.take<int32_t>(1);
  f.tiles = cv.take<int4>(moe::mfma_tiles_max(T, c.top_k, c.n_experts, c.n_shared));
  f.h = cv.take<float>(pairs * c.inter);
  f.qh_rows = cv.take<int8_t>(act_rows(c) ? pairs * c.inter : 0);
  f.dh_rows = cv.take<float>(act_rows(c) ? pairs : 0);
  return f;
}

struct LayerWs {
  float *ssq;
  int32_t *slots;
  float *hs;
  RouteWs route;
  int32_t *idx;
  float *w;
  int8_t *q;
  float *d;
  float *expert_out, *shared_out;
  int8_t *qh;
  float *dh;
  FfnWs ffn;
};
LayerWs carve_layer(Carve &cv, const moe_cfg &c, int T) {
  LayerWs l;
  l.ssq = cv.take<float>((size_t)T * (c.hidden / 8));
  l.slots = cv.take<int32_t>(moe::small_batch_slot_ints(T, c.top_k, c.n_shared));
  l.hs = cv.take<float>((size_t)T * c.inter * c.n_shared);
  l.route = carve_route(cv, c, T);
  l.idx = cv.take<int32_t>((size_t)T * c.top_k);
  l.w = cv.take<float>((size_t)T * c.top_k);
  l.q = cv.take<int8_t>((size_t)T * c.hidden);
  l.d = cv.take<float>((size_t)T * c.hidden / 32);
  l.expert_out = cv.take<float>((size_t)T * c.top_k * c.hidden);
  l.shared_out = cv.take<float>((size_t)T * c.hidden * c.n_shared);
  const size_t pairs = (size_t)T * c.top_k + (size_t)T * c.n_shared;
  l.qh = cv.take<int8_t>(pairs * c.inter);
  l.dh = cv.take<float>(pairs * (c.inter / 32));
  l.ffn = carve_ffn(cv, c, T);
  return l;
}

// unchecked enqueue helpers (arguments validated by the callers) ------------
int do_route(const moe_cfg &c, int T, const float *x, const float *wr, const float *bias,
             int32_t *idx, float *w, const RouteWs &ws, hipStream_t st,
             const moe_events *ev = nullptr) {
  moe::launch_router_scores(c, T, x, wr, bias, ws.s, ws.sb, st, ev);
  moe::launch_router_select(c, T, ws.s, ws.sb, idx, w, st, ev);
  return launched("moe_route");
}

int do_ffn(const moe_cfg &c, int T, const int8_t *q, const float *d, const int32_t *idx,
           const void *experts, const void *shared, float *expert_out, float *shared_out,
           const FfnWs &ws, const moe_ffn_debug *dbg, hipStream_t st,
           const moe_events *ev = nullptr, const void *const *expert_ptrs = nullptr) {
  moe::launch_group(T * c.top_k, c.n_experts, idx, ws.counts, ws.offsets, ws.perm, ws.inv,
                    ws.active, ws.n_active, st, ev);
  moe::FfnArgs a;
  a.H = c.hidden;
  a.I = c.inter;
  a.E = c.n_experts;
  a.K = c.top_k;
  a.T = T;
  a.n_shared = c.n_shared;
  a.wbits = c.wbits;
  a.wfmt = c.wfmt;
  a.blob_bytes = blob_bytes(c);
  a.q = q;
  a.d = d;
  a.experts = static_cast<const uint8_t *>(experts);
  a.expert_ptrs = reinterpret_cast<const uint8_t *const *>(expert_ptrs);
  a.shared = static_cast<const uint8_t *>(shared);
  a.offsets = ws.offsets;
  a.perm = ws.perm;
  a.active = ws.active;
  a.n_active = ws.n_active;
  a.h = ws.h;
  a.expert_out = expert_out;
  a.shared_out = shared_out;
  if (dbg) a.dbg = *dbg;
  else memset(&a.dbg, 0, sizeof(a.dbg));
  if (act_rows(c)) {  // per-row activation scales: the row-dot MFMA kernels at every T
    if (!moe::mfma_rows_supported(a))
      return fail(MOE_EINVAL, "per-row activations need hidden and inter multiples of 128");
    int8_t *q_h = a.dbg.q_h ? a.dbg.q_h : ws.qh_rows;  // written straight into a dump
    float *d_h = a.dbg.d_h ? a.dbg.d_h : ws.dh_rows;
    moe::launch_ffn_mfma_rows(a, ws.tiles, ws.n_tiles, ws.h, q_h, d_h, idx, st, ev);
    return launched("moe_expert_ffn");
  }
  if (c.wfmt == 2) {  // FP8: the vector kernels with exact block dots, every T
    if (!moe::f8_supported(a))
      return fail(MOE_EINVAL, "FP8 experts need hidden <= 8192 and inter <= 4096");
    moe::launch_ffn_f8(a, st, ev);
    return launched("moe_expert_ffn");
  }
  const bool mfma = moe::mfma_supported(a);
  const bool mfma_only = c.wbits == 8 || c.wfmt == 1;  // the vector-dot kernels take int4/int2
  if (mfma_only && !mfma)
    return fail(MOE_EINVAL, "int8 / MXFP4 experts need the matrix-core path (H %% 256, I %% 64)");
  if ((T >= MOE_MFMA_MIN_T || mfma_only) && mfma) {  // grouped GEMMs, matrix cores
    const size_t pairs = (size_t)T * c.top_k + (size_t)T * c.n_shared;
    int8_t *q_h = reinterpret_cast<int8_t *>(ws.h);
    float *d_h = reinterpret_cast<float *>(q_h + ((pairs * c.inter + 255) & ~(size_t)255));
    moe::launch_ffn_mfma(a, ws.tiles, ws.n_tiles, q_h, d_h, st, ev);
  } else {
    moe::launch_ffn_gemv(a, st, ev);
  }
  return launched("moe_expert_ffn");
}

}  // namespace

extern "C" {

size_t moe_expert_blob_bytes(const moe_cfg *cfg) {
  if (check_cfg(cfg) != MOE_OK) return 0;
  return blob_bytes(*cfg);
}

size_t moe_route_workspace(const moe_cfg *cfg, int32_t T) {
  if (check_cfg(cfg) != MOE_OK || T < 0) return 0;
  Carve cv{nullptr};
  carve_route(cv, *cfg, T);
  return cv.off;
}

int moe_route(const moe_cfg *cfg, int32_t T, const float *x, const float *w_router,
              const float *bias, int32_t *idx, float *w, void *workspace, size_t ws_bytes,
              void *stream) {
  clear_hip_error();  // MOE_EHIP then names this call's own launches
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T=%d < 0", T);
  if (T == 0) return MOE_OK;
  REQUIRE(x, "x");
  REQUIRE(w_router, "w_router");
  REQUIRE(bias, "bias");
  REQUIRE(idx, "idx");
  REQUIRE(w, "w");
  const size_t need = moe_route_workspace(cfg, T);
  if (!workspace || ws_bytes < need)
    return fail(MOE_EWORKSPACE, "route workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(workspace, 256)) return fail(MOE_EALIGN, "workspace is not 256-byte aligned");
  Carve cv{static_cast<uint8_t *>(workspace)};
  RouteWs ws = carve_route(cv, *cfg, T);
  return do_route(*cfg, T, x, w_router, bias, idx, w, ws, (hipStream_t)stream);
}

int moe_quant_act(int32_t rows, int32_t n, int32_t block, const float *x, int8_t *q, float *d,
                  void *stream) {
  clear_hip_error();  // MOE_EHIP then names this call's own launches
  if (rows < 0) return fail(MOE_EINVAL, "rows=%d < 0", rows);
  if (n <= 0 || n % 32) return fail(MOE_EINVAL, "n=%d must be a positive multiple of 32", n);
  if (block != 32 && block != n)
    return fail(MOE_EINVAL, "block=%d must be 32 (Q8_0) or n=%d (one scale per row)", block, n);
  if (rows == 0) return MOE_OK;
  REQUIRE(x, "x");
  REQUIRE(q, "q");
  REQUIRE(d, "d");
  if (block == 32) moe::launch_quant_act(x, q, d, (int64_t)rows * n, (hipStream_t)stream);
  else moe::launch_quant_rows(x, q, d, rows, n, nullptr, 0, (hipStream_t)stream);
  return launched("moe_quant_act");
}

int moe_group(const moe_cfg *cfg, int32_t T, const int32_t *idx, int32_t *counts,
              int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active,
              int32_t *n_active, void *stream) {
  clear_hip_error();  // MOE_EHIP then names this call's own launches
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T=%d < 0", T);
  if (T == 0) return MOE_OK;
  REQUIRE(idx, "idx");
  REQUIRE(counts, "counts");
  REQUIRE(offsets, "offsets");
  REQUIRE(perm, "perm");
  REQUIRE(inv, "inv");
  REQUIRE(active, "active");
  REQUIRE(n_active, "n_active");
  moe::launch_group(T * cfg->top_k, cfg->n_experts, idx, counts, offsets, perm, inv, active,
                    n_active, (hipStream_t)stream);
  return launched("moe_group");
}

size_t moe_expert_ffn_workspace(const moe_cfg *cfg, int32_t T) {
  if (check_cfg(cfg) != MOE_OK || T < 0) return 0;
  Carve cv{nullptr};
  carve_ffn(cv, *cfg, T);
  return cv.off;
}

int moe_expert_ffn(const moe_cfg *cfg, int32_t T, const int8_t *q, const float *d,
                   const int32_t *idx, const void *experts, const void *shared,
                   float *expert_out, float *shared_out, void *workspace, size_t ws_bytes,
                   const moe_ffn_debug *dbg, void *stream) {
  clear_hip_error();  // MOE_EHIP then names this call's own launches
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T=%d < 0", T);
  if (T == 0) return MOE_OK;
  REQUIRE(q, "q");
  REQUIRE(d, "d");
  REQUIRE(idx, "idx");
  REQUIRE(experts, "experts");
  REQUIRE(expert_out, "expert_out");
  if (!aligned(experts, 256)) return fail(MOE_EALIGN, "experts is not 256-byte aligned");
  if (cfg->n_shared) {
    REQUIRE(shared, "shared");
    REQUIRE(shared_out, "shared_out");
    if (!aligned(shared, 256)) return fail(MOE_EALIGN, "shared is not 256-byte aligned");
  }
  if (dbg) {
    OPTIONAL(dbg->gate_dots, "dbg->gate_dots");
    OPTIONAL(dbg->up_dots, "dbg->up_dots");
    OPTIONAL(dbg->h, "dbg->h");
    OPTIONAL(dbg->q_h, "dbg->q_h");
    OPTIONAL(dbg->d_h, "dbg->d_h");
    OPTIONAL(dbg->down_dots, "dbg->down_dots");
  }
  const size_t need = moe_expert_ffn_workspace(cfg, T);
  if (!workspace || ws_bytes < need)
    return fail(MOE_EWORKSPACE, "ffn workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(workspace, 256)) return fail(MOE_EALIGN, "workspace is not 256-byte aligned");
  Carve cv{static_cast<uint8_t *>(workspace)};
  FfnWs ws = carve_ffn(cv, *cfg, T);
  return do_ffn(*cfg, T, q, d, idx, experts, cfg->n_shared ? shared : nullptr, expert_out,
                cfg->n_shared ? shared_out : nullptr, ws, dbg, (hipStream_t)stream);
}

int moe_combine(int32_t T, int32_t H, int32_t K, const float *expert_out, const float *w,
                const float *shared_out, const float *residual, float *y, float *y_norm,
                float eps, void *stream) {
  clear_hip_error();  // MOE_EHIP then names this call's own launches
  if (T < 0) return fail(MOE_EINVAL, "T=%d < 0", T);
  if (H <= 0 || H % 4) return fail(MOE_EINVAL, "H=%d must be a positive multiple of 4", H);
  if (K < 0 || K > 16) return fail(MOE_EINVAL, "K=%d not in [0,16]", K);
  if (!(eps >= 0.0f)) return fail(MOE_EINVAL, "eps must be >= 0");
  if (T == 0) return MOE_OK;
  if (K > 0) {
    REQUIRE(expert_out, "expert_out");
    REQUIRE(w, "w");
  }
  OPTIONAL(shared_out, "shared_out");
  OPTIONAL(residual, "residual");
  REQUIRE(y, "y");
  OPTIONAL(y_norm, "y_norm");
  const size_t row_bytes = sizeof(float) * (size_t)T * H;
  if (overlap(y, row_bytes, y_norm, row_bytes))
    return fail(MOE_EINVAL, "y_norm overlaps y");
  moe::launch_combine(T, H, K, expert_out, w, shared_out, residual, y, y_norm, eps,
                      (hipStream_t)stream);
  return launched("moe_combine");
}

int moe_mfma_peak(int32_t n_wg, int32_t iters, int32_t *out, void *stream) {
  clear_hip_error();  // MOE_EHIP then names this call's own launches
  if (n_wg <= 0 || n_wg > (1 << 20)) return fail(MOE_EINVAL, "n_wg=%d not in [1, 2^20]", n_wg);
  if (iters <= 0 || iters >= (1 << 21)) return fail(MOE_EINVAL, "iters=%d not in [1, 2^21)", iters);
  REQUIRE(out, "out");
  moe::launch_mfma_peak(n_wg, iters, out, (hipStream_t)stream);
  return launched("moe_mfma_peak");
}

int moe_read_peak(const void *buf, int64_t bytes, int32_t n_wg, uint32_t *out, void *ev_start,
                  void *ev_stop, void *stream) {
  clear_hip_error();  // MOE_EHIP then names this call's own launches
  if (bytes <= 0 || bytes % 16)
    return fail(MOE_EINVAL, "bytes=%lld must be a positive multiple of 16", (long long)bytes);
  if (n_wg <= 0 || n_wg > (1 << 20)) return fail(MOE_EINVAL, "n_wg=%d not in [1, 2^20]", n_wg);
  REQUIRE(buf, "buf");
  REQUIRE(out, "out");
  moe::Ev ev;
  ev.start = (hipEvent_t)ev_start;
  ev.stop = (hipEvent_t)ev_stop;
  moe::launch_read_peak(buf, bytes, n_wg, out, (hipStream_t)stream, ev);
  return launched("moe_read_peak");
}

int moe_rmsnorm(int32_t T, int32_t H, const float *x, float *y, float eps, void *stream) {
  clear_hip_error();  // MOE_EHIP then names this call's own launches
  if (T < 0) return fail(MOE_EINVAL, "T=%d < 0", T);
  if (H <= 0 || H % 4) return fail(MOE_EINVAL, "H=%d must be a positive multiple of 4", H);
  if (!(eps >= 0.0f)) return fail(MOE_EINVAL, "eps must be >= 0");
  if (T == 0) return MOE_OK;
  REQUIRE(x, "x");
  REQUIRE(y, "y");
  const size_t row_bytes = sizeof(float) * (size_t)T * H;
  if (overlap(x, row_bytes, y, row_bytes)) return fail(MOE_EINVAL, "y overlaps x");
  moe::launch_rmsnorm(T, H, x, y, eps, (hipStream_t)stream);
  return launched("moe_rmsnorm");
}

size_t moe_layer_workspace(const moe_cfg *cfg, int32_t T) {
  if (check_cfg(cfg) != MOE_OK || T < 0) return 0;
  Carve cv{nullptr};
  carve_layer(cv, *cfg, T);
  return cv.off;
}

}  // extern "C"

namespace {

// moe_layer with the routed records either contiguous (experts) or given one
// pointer each (expert_ptrs, a device array of E pointers); exactly one is set.
bool any_ffn_dump(const moe_ffn_debug &f) {
  return f.gate_dots || f.up_dots || f.h || f.q_h || f.d_h || f.down_dots;
}

int check_layer_debug(const moe_layer_debug *g) {
  if (!g) return MOE_OK;
  OPTIONAL(g->q, "dbg->q");
  OPTIONAL(g->d, "dbg->d");
  const int32_t *u[6] = {g->counts, g->offsets, g->perm, g->inv, g->active, g->n_active};
  const char *un[6] = {"dbg->counts", "dbg->offsets", "dbg->perm", "dbg->inv", "dbg->active",
                       "dbg->n_active"};
  int given = 0;
  for (int i = 0; i < 6; i++) {
    OPTIONAL(u[i], un[i]);
    given += u[i] != nullptr;
  }
  if (given != 0 && given != 6)
    return fail(MOE_EINVAL, "dbg: the six union arrays are given together or not at all");
  OPTIONAL(g->ffn.gate_dots, "dbg->ffn.gate_dots");
  OPTIONAL(g->ffn.up_dots, "dbg->ffn.up_dots");
  OPTIONAL(g->ffn.h, "dbg->ffn.h");
  OPTIONAL(g->ffn.q_h, "dbg->ffn.q_h");
  OPTIONAL(g->ffn.d_h, "dbg->ffn.d_h");
  OPTIONAL(g->ffn.down_dots, "dbg->ffn.down_dots");
  return MOE_OK;
}

int layer_impl(const moe_cfg *cfg, int32_t T, const float *x, const float *w_router,
               const float *bias, const void *experts, const void *const *expert_ptrs,
               const void *shared, const float *residual, float *y, float *y_norm, float eps,
               int32_t *idx_out, float *w_out, void *workspace, size_t ws_bytes,
               const moe_events *ev, const moe_layer_debug *dbg, void *stream) {
  clear_hip_error();  // MOE_EHIP then names this call's own launches
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T=%d < 0", T);
  if (!(eps >= 0.0f)) return fail(MOE_EINVAL, "eps must be >= 0");
  if (T == 0) return MOE_OK;
  REQUIRE(x, "x");
  REQUIRE(w_router, "w_router");
  REQUIRE(bias, "bias");
  REQUIRE(y, "y");
  OPTIONAL(residual, "residual");
  OPTIONAL(y_norm, "y_norm");
  OPTIONAL(idx_out, "idx_out");
  OPTIONAL(w_out, "w_out");
  if (overlap(y, sizeof(float) * (size_t)T * cfg->hidden, y_norm,
              sizeof(float) * (size_t)T * cfg->hidden))
    return fail(MOE_EINVAL, "y_norm overlaps y");
  if (expert_ptrs) {
    if (!aligned(expert_ptrs, 8)) return fail(MOE_EALIGN, "expert_ptrs is not 8-byte aligned");
  } else {
    REQUIRE(experts, "experts");
    if (!aligned(experts, 256)) return fail(MOE_EALIGN, "experts is not 256-byte aligned");
  }
  if (cfg->n_shared) {
    REQUIRE(shared, "shared");
    if (!aligned(shared, 256)) return fail(MOE_EALIGN, "shared is not 256-byte aligned");
  }
  if ((rc = check_layer_debug(dbg))) return rc;
  moe_layer_debug g;
  if (dbg) g = *dbg;
  else memset(&g, 0, sizeof(g));
  const bool dump_union = g.counts != nullptr, dump_ffn = any_ffn_dump(g.ffn);
  const size_t need = moe_layer_workspace(cfg, T);
  if (!workspace || ws_bytes < need)
    return fail(MOE_EWORKSPACE, "layer workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(workspace, 256)) return fail(MOE_EALIGN, "workspace is not 256-byte aligned");
  const moe_cfg &c = *cfg;
  hipStream_t st = (hipStream_t)stream;
  Carve cv{static_cast<uint8_t *>(workspace)};
  LayerWs ws = carve_layer(cv, c, T);
  int32_t *idx = idx_out ? idx_out : ws.idx;
  float *w = w_out ? w_out : ws.w;
  int8_t *q = g.q ? g.q : ws.q;  // the kernels write Q8_0 of x straight into a dump
  float *d = g.d ? g.d : ws.d;
  if (!act_rows(c) && moe::small_batch_supported(c, T)) {
    moe::LayerArgs a;
    a.H = c.hidden;
    a.I = c.inter;
    a.E = c.n_experts;
    a.G = c.n_group;
    a.TG = c.topk_group;
    a.K = c.top_k;
    a.T = T;
    a.n_shared = c.n_shared;
    a.wbits = c.wbits;
    a.wfmt = c.wfmt;
    a.scale = c.routed_scaling;
    a.top_p = c.top_p;
    a.eps = eps;
    a.blob_bytes = blob_bytes(c);
    a.x = x;
    a.wr = w_router;
    a.bias = bias;
    a.residual = residual;
    a.experts = static_cast<const uint8_t *>(experts);
    a.expert_ptrs = reinterpret_cast<const uint8_t *const *>(expert_ptrs);
    a.shared = c.n_shared ? static_cast<const uint8_t *>(shared) : nullptr;
    a.y = y;
    a.y_norm = y_norm;
    a.idx = idx;
    a.w = w;
    a.s = ws.route.s;
    a.sb = ws.route.sb;
    a.q = q;
    a.d = d;
    a.slots = ws.slots;
    a.hs = ws.hs;
    a.qh = ws.qh;
    a.dh = ws.dh;
    a.ssq = ws.ssq;
    a.eo_r = ws.expert_out;
    a.eo_s = c.n_shared ? ws.shared_out : nullptr;
    a.dbg = g;
    if (dump_union || dump_ffn) moe::launch_small_batch_dbg(a, st, ev);
    else moe::launch_small_batch(a, st, ev);
    return launched("moe_layer (small batch)");
  }
  if ((rc = do_route(c, T, x, w_router, bias, idx, w, ws.route, st, ev))) return rc;
  if (act_rows(c)) moe::launch_quant_rows(x, q, d, T, c.hidden, nullptr, 0, st, ev);
  else moe::launch_quant_act(x, q, d, (int64_t)T * c.hidden, st, ev);
  if ((rc = launched("moe_layer quant"))) return rc;
  FfnWs fws = ws.ffn;
  if (dump_union) {  // the grouping kernel writes the union straight into the dump
    fws.counts = g.counts;
    fws.offsets = g.offsets;
    fws.perm = g.perm;
    fws.inv = g.inv;
    fws.active = g.active;
    fws.n_active = g.n_active;
  }
  if ((rc = do_ffn(c, T, q, d, idx, experts, c.n_shared ? shared : nullptr, ws.expert_out,
                   c.n_shared ? ws.shared_out : nullptr, fws, dump_ffn ? &g.ffn : nullptr, st,
                   ev, expert_ptrs)))
    return rc;
  moe::launch_combine(T, c.hidden, c.top_k, ws.expert_out, w,
                      c.n_shared ? ws.shared_out : nullptr, residual, y, y_norm, eps, st, ev);
  return launched("moe_layer combine");
}

}  // namespace

extern "C" {

int moe_layer(const moe_cfg *cfg, int32_t T, const float *x, const float *w_router,
              const float *bias, const void *experts, const void *shared,
              const float *residual, float *y, float *y_norm, float eps, int32_t *idx_out,
              float *w_out, void *workspace, size_t ws_bytes, const moe_events *ev,
              const moe_layer_debug *dbg, void *stream) {
  if (!experts) return fail(MOE_EINVAL, "experts is NULL");
  return layer_impl(cfg, T, x, w_router, bias, experts, nullptr, shared, residual, y, y_norm,
                    eps, idx_out, w_out, workspace, ws_bytes, ev, dbg, stream);
}

int moe_layer_ptrs(const moe_cfg *cfg, int32_t T, const float *x, const float *w_router,
                   const float *bias, const void *const *expert_ptrs, const void *shared,
                   const float *residual, float *y, float *y_norm, float eps, int32_t *idx_out,
                   float *w_out, void *workspace, size_t ws_bytes, const moe_events *ev,
                   const moe_layer_debug *dbg, void *stream) {
  if (!expert_ptrs) return fail(MOE_EINVAL, "expert_ptrs is NULL");
  return layer_impl(cfg, T, x, w_router, bias, nullptr, expert_ptrs, shared, residual, y, y_norm,
                    eps, idx_out, w_out, workspace, ws_bytes, ev, dbg, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- moe_layer_noalloc

// The workspace of moe_layer_noalloc: one copy per device (each device that
// runs the library holds its own until the process ends), shared by every
// call on that device.  In host code `scratch` names a host-side stand-in,
// not device memory: the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// handed to kernels.  No call needs any of it zeroed (every byte a call
// reads it wrote earlier in the same call).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the scratch array on the device of `st` (the current
// device for the null stream).
int scratch_of(hipStream_t st, void **out) {
  int dev = -1;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_EHIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EINVAL, "device %d out of range", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    hipError_t r = hipGetDevice(&cur);
    if (r == hipSuccess && cur != dev) r = hipSetDevice(dev);
    void *p = nullptr;
    if (r == hipSuccess) r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
    g_scratch_ptr[dev] = p;
    g_scratch_err[dev] = r;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return fail(MOE_EHIP, "scratch of device %d: %s", dev,
                hipGetErrorString(g_scratch_err[dev] != hipSuccess ? g_scratch_err[dev]
                                                                    : hipErrorInvalidSymbol));
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_noalloc(const moe_cfg *cfg, int32_t T, const float *x, const float *w_router,
                      const float *bias, const void *experts, const void *shared,
                      const float *residual, float *y, float *y_norm, float eps,
                      int32_t *idx_out, float *w_out, const moe_events *ev, void *stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T=%d < 0", T);
  if (T == 0) return MOE_OK;
  const size_t need = moe_layer_workspace(cfg, T);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_EWORKSPACE,
                "moe_layer_noalloc: %d tokens need %zu bytes of workspace, more than its %u-byte "
                "scratch (use moe_layer with a workspace)",
                T, need, (unsigned)MOE_NOALLOC_SCRATCH_BYTES);
  if (!experts) return fail(MOE_EINVAL, "experts is NULL");
  void *ws = nullptr;
  if ((rc = scratch_of((hipStream_t)stream, &ws))) return rc;
  return layer_impl(cfg, T, x, w_router, bias, experts, nullptr, shared, residual, y, y_norm, eps,
                    idx_out, w_out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, ev, nullptr, stream);
}

const char *moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EALIGN: return "misaligned pointer";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch failure";
    default: return "unknown error";
  }
}

const char *moe_last_error(void) { return g_msg; }

}  // extern "C"

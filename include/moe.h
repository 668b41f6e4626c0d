/*
 * libmoe — one routed Mixture-of-Experts layer step on an AMD MI355X (gfx950).
 *
 * The step, as the pages describe it ("Show HN: 遅いコンピュータで GLM 5.2 を
 * 実行する", ja.news.hada.io, section 実装済みの主な機能; "Comment exécuter un
 * réseau de neurones de 744 milliards de paramètres sur un ordinateur
 * ordinaire", devtrends.cc, section "Comment fonctionne le moteur"):
 *   1. a DeepSeek-V3-style sigmoid router with noaux_tc group-limited top-k,
 *      routed_scaling_factor, and a shared expert;
 *   2. Q8_0-style int8 activations;
 *   3. batch union: each distinct expert selected by a batch is read once and
 *      applied to every token routed to it;
 *   4. expert FFNs whose three matrices are packed int4 (or int2) codes with
 *      one scale per row, dequantised on use, multiplied against the int8
 *      activations with exact integer accumulation;
 *   5. the weighted sum of the routed experts plus the shared expert.
 *
 * Conventions for every call:
 *   - cfg (and any moe_ffn_debug / moe_layer_debug struct) is a host
 *     pointer; every other pointer is a
 *     DEVICE pointer to caller-owned memory, at least 16-byte aligned.
 *   - The library never allocates or frees device memory and never copies
 *     between host and device.  Scratch memory comes from a caller-provided
 *     workspace whose size is given by the matching *_workspace() query.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream), in order, without host synchronisation.  Returning 0 means
 *     the work was enqueued; device-side faults surface at the caller's next
 *     synchronisation, as for any HIP call.
 *   - On a non-zero return nothing has been enqueued.  moe_strerror() names
 *     the code; moe_last_error() gives a per-thread message with details.
 *     A call that launches work first clears HIP's per-thread last-error
 *     state (hipGetLastError), so MOE_EHIP always describes a failure of
 *     that call's own launches, never an earlier failed HIP call of the
 *     caller's.
 *   - T = 0 tokens is a valid no-op.
 *   - Results are bit-identical from run to run for fixed inputs and device
 *     (no floating-point atomics).
 *   - Calls are reentrant; they keep no state beyond the per-thread message.
 *
 * Data layouts (row-major):
 *   x        fp32 [T][H]        token hidden states
 *   w_router fp32 [E][H]        router matrix, one row per routed expert
 *   bias     fp32 [E]           noaux_tc correction bias (selection only)
 *   idx      int32 [T][K]       selected experts, rank order
 *   w        fp32 [T][K]        routing weights, rank order
 *   q, d     int8 [T][n], fp32 [T][n/32]   Q8_0 codes and block scales
 *   expert records: moe_expert_blob_bytes(cfg) bytes per expert, routed
 *     expert e at experts + e * blob_bytes; layout of one record:
 *       gate codes [I][H*wbits/8] | up codes [I][H*wbits/8] |
 *       down codes [H][I*wbits/8] | gate scale fp32 [I] | up scale fp32 [I] |
 *       down scale fp32 [H]
 *     MXFP4 records (wfmt = 1; "Comment exécuter…", section "Modèles
 *     supportés": native MXFP4 weights): the codes as for int4 but FP4 E2M1
 *     (sign bit 3, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6), then one E8M0 byte
 *     s per 32 consecutive codes of a row (value 2^(s-127)) instead of the
 *     row scales: gate [I][H/32] | up [I][H/32] | down [H][I/32]; a row is
 *     sum_b 2^(s_b-127) d_b sum_k fp4(c_k) q_k, and the int32 block dot
 *     reported for it (moe_ffn_debug) is sum_k 2 fp4(c_k) q_k.
 *     FP8 records (wfmt = 2, wbits 8; "Comment exécuter…", section "Modèles
 *     supportés": a supported model runs on fp4/fp8 weights, and "Show
 *     HN…", converter item: FP8 checkpoints with 128x128 block scales): one
 *     OCP FP8 E4M3 byte per element (bias 7, 3 mantissa bits, largest 448;
 *     codes 0x7F and 0xFF are NaN and not valid weights) for gate [I][H],
 *     up [I][H], down [H][I], then one fp32 scale per 128x128 block: gate
 *     [I/128][H/128] | up [I/128][H/128] | down [H/128][I/128]; a row r is
 *     sum_b S[r/128][b/4] d_b sum_k fp8(c_k) q_k over its 32-blocks b, and
 *     the int32 block dot reported for it is sum_k 512 fp8(c_k) q_k (exact:
 *     512 fp8 is an integer).  hidden and inter multiples of 128;
 *     moe_expert_ffn runs vector kernels at every batch size (no
 *     matrix-core path); moe_layer takes the small-batch kernels up to 4
 *     tokens and the chained kernels above.
 *     int8: element j in byte j, codes in [-127, 127] (-128 is not
 *     produced by the quantiser but is accepted);
 *     int4: element 2j in the low nibble of byte j, 2j+1 in the high nibble;
 *     int2: element 4j+i in bits 2i..2i+1; codes are two's complement and
 *     every bit pattern is a valid code.  Weight value = scale[row] * code.
 *     The blob base pointer must be 256-byte aligned (so is every record,
 *     since blob_bytes is a multiple of 256 for supported shapes).
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOE_OK 0
#define MOE_EINVAL (-1)     /* bad shape, count or null required pointer */
#define MOE_EALIGN (-2)     /* pointer not aligned as documented */
#define MOE_EWORKSPACE (-3) /* workspace missing or smaller than required */
#define MOE_EHIP (-4)       /* a HIP launch failed; see moe_last_error() */

/* Layer shape.  Supported: hidden % 256 == 0, inter % 128 == 0,
 * 2 <= n_experts <= 1024, n_experts % n_group == 0 with at least 2 experts
 * per group, n_group <= 64, 1 <= topk_group <= n_group,
 * 1 <= top_k <= min(16, topk_group * n_experts / n_group), n_shared in {0,1},
 * wbits in {8, 4, 2}; a weight row holds at most 256 16-byte pieces of codes
 * (448 for int8) along hidden and 128 along inter, i.e. hidden <= 8192 and
 * inter <= 4096 for int4 (16384 / 8192 for int2, 7168 / 2048 for int8);
 * top_p = 0 (off), or in (0, 1] (1 is off as well); wfmt 0, 1 with
 * wbits 4 (MXFP4), or 2 with wbits 8 (FP8); act_block 0 or 32 (Q8_0), or
 * MOE_ACT_ROW with int4 or int8 codes (wfmt 0). */
/* Activation format act_block = MOE_ACT_ROW: one fp32 scale per activation
 * row instead of one per 32 values -- per token row of x (H values) and per
 * (token, expert) row of h (I values) -- with the Q8_0 rule over the whole
 * row: d = amax/127, q = clamp(roundf(x * (1/d)), -127, 127).  An output
 * row is then scale_r * d * P with P the exact int32 dot over the whole row
 * (a second format beside the pages' Q8_0 blocks, "Show HN…", 実装済みの主な
 * 機能, integer-dot item; with one integer accumulator per row the matrix
 * cores run without per-block scaling).  q and d of x are then int8 [T][H]
 * and fp32 [T]. */
#define MOE_ACT_ROW (-1)
typedef struct moe_cfg {
  int32_t hidden;       /* H */
  int32_t inter;        /* I, intermediate width of every expert (shared too) */
  int32_t n_experts;    /* E, routed experts */
  int32_t n_group;      /* G, expert groups for group-limited routing */
  int32_t topk_group;   /* TG, groups kept per token */
  int32_t top_k;        /* K, routed experts per token */
  int32_t n_shared;     /* 0 or 1 shared expert */
  int32_t wbits;        /* 8 (int8), 4 (packed int4) or 2 (packed int2) */
  float routed_scaling; /* routed_scaling_factor applied to routed weights */
  float top_p;          /* adaptive expert top-p (see moe_route); 0 = off */
  int32_t wfmt;         /* 0: integer codes, fp32 row scales; 1: MXFP4 (wbits 4);
                           2: FP8 E4M3 with 128x128 block scales (wbits 8) */
  int32_t act_block;    /* activations: 0 or 32 = Q8_0 blocks; MOE_ACT_ROW = one scale per row */
} moe_cfg;

/* Bytes of one packed expert record for cfg (0 if cfg is unsupported). */
size_t moe_expert_blob_bytes(const moe_cfg *cfg);

/* ---------------------------------------------------------------------------
 * moe_route — router ("Show HN…", 実装済みの主な機能, router item: sigmoid
 * scores, noaux_tc, routed_scaling_factor).
 *   s[t,e]  = sigmoid(x[t] . w_router[e]), computed in fp32 in one fixed order:
 *             the dot product runs over consecutive chunks of 64 elements,
 *             each an fma chain in increasing index from 0, chunk partials added
 *             left to right; e^y uses Cody–Waite reduction by ln 2 and a
 *             degree-7 Taylor polynomial (fma Horner), then scaling by 2^n;
 *             sigmoid(l) = 1 / (1 + e^-l).
 *   sb[t,e] = s[t,e] + bias[e]                    (bias used for selection only)
 *   group score = sum of the two largest sb in each of the G contiguous groups;
 *   the TG best groups are kept (ties: lower group index); the K best experts
 *   of the kept groups by sb (ties: lower expert index) are written to idx in
 *   rank order; w[t,k] = (s[t,idx] / S) * routed_scaling with
 *   S = sum_k s[t,idx[t,k]] added in rank order (fp32).
 * Adaptive expert top-p ("Show HN…", section モデルのダウンロードと実行,
 * options list: an expert top-p that cuts expert reads), when 0 < top_p < 1:
 * with c_j = s_0 + ... + s_j added in rank order (fp32) and thr = top_p * S
 * (fp32), the first n ranks are kept, n = 1 + the first j with c_j >= thr;
 * their weights become w = (s / c_{n-1}) * routed_scaling and the other
 * ranks get idx = -1 and w = 0 (no later call reads an expert for them).
 * idx and w are bit-identical to a CPU implementation of the same steps.
 * workspace: >= moe_route_workspace(cfg, T) bytes (may be NULL if that is 0).
 * Errors: MOE_EINVAL (cfg, T < 0, null pointer), MOE_EALIGN, MOE_EWORKSPACE.
 * ------------------------------------------------------------------------- */
size_t moe_route_workspace(const moe_cfg *cfg, int32_t T);
int moe_route(const moe_cfg *cfg, int32_t T, const float *x, const float *w_router,
              const float *bias, int32_t *idx, float *w, void *workspace, size_t ws_bytes,
              void *stream);

/* ---------------------------------------------------------------------------
 * moe_quant_act — Q8_0-style int8 activations ("Show HN…", 実装済みの主な機能,
 * integer-dot item).  For each of `rows` rows of n floats and each block of
 * `block` values (32: Q8_0; n: one scale per row, the MOE_ACT_ROW format):
 *   d = amax / 127 (fp32, correctly rounded), id = d != 0 ? 1/d : 0,
 *   q = clamp(roundf(x * id), -127, 127)  (round half away from zero).
 * q int8 [rows][n], d fp32 [rows][n/block].
 * Bit-identical to the same steps on a CPU.  n % 32 == 0.
 * Errors: MOE_EINVAL (rows < 0, n <= 0 or n % 32, block not 32 or n, null
 * pointer), MOE_EALIGN.
 * ------------------------------------------------------------------------- */
int moe_quant_act(int32_t rows, int32_t n, int32_t block, const float *x, int8_t *q, float *d,
                  void *stream);

/* ---------------------------------------------------------------------------
 * moe_group — batch-union grouping ("Show HN…", 実装済みの主な機能, batch-union
 * MoE item; devtrends, "Comment fonctionne le moteur": duplicate requests
 * for one expert are merged).  Slots s = t*K + k of idx [T][K]:
 *   counts[e]   number of slots routed to e                       int32 [E]
 *   offsets[e]  exclusive prefix sum of counts; offsets[E] = number
 *               of routed slots (T*K unless top-p dropped some)   int32 [E+1]
 *   perm        slots grouped by expert, increasing slot (= token) order
 *               inside each expert, then -1 up to T*K             int32 [T*K]
 *   inv[s]      position of slot s in perm, -1 if not routed      int32 [T*K]
 *   active      experts with counts > 0, ascending, then -1       int32 [E]
 *   n_active    number of such experts                            int32 [1]
 * idx entries outside [0, E) (-1: dropped by top-p) are not routed.
 * Bit-identical to a stable counting sort on the CPU.
 * Errors: MOE_EINVAL (cfg, T < 0, null pointer), MOE_EALIGN.
 * ------------------------------------------------------------------------- */
int moe_group(const moe_cfg *cfg, int32_t T, const int32_t *idx, int32_t *counts,
              int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active,
              int32_t *n_active, void *stream);

/* Optional device buffers a test can pass to moe_expert_ffn to receive the
 * intermediate results (any member may be NULL; pass NULL for the struct in
 * production).  Pair p < T*K is slot p (token p / K, rank p % K); pair
 * T*K + t is the shared expert applied to token t.  P = T*K + T*n_shared.
 * B = 32 for Q8_0 activations, the row length for MOE_ACT_ROW (one dot per
 * output row):
 *   gate_dots, up_dots  int32 [P][I][H/B]  exact block dots of code . q
 *   h                   fp32  [P][I]       silu(gate) * up
 *   q_h, d_h            int8 [P][I], fp32 [P][I/B]   activations of h
 *   down_dots           int32 [P][H][I/B]  exact block dots of code . q_h   */
typedef struct moe_ffn_debug {
  int32_t *gate_dots;
  int32_t *up_dots;
  float *h;
  int8_t *q_h;
  float *d_h;
  int32_t *down_dots;
} moe_ffn_debug;

/* ---------------------------------------------------------------------------
 * moe_expert_ffn — the routed and shared expert FFNs ("Show HN…",
 * 実装済みの主な機能: quantisation-kernel item, packed int4/int2 with per-row
 * scales, dequantised on use; integer-dot item; batch-union item).
 * For each selected (token t, expert e) and for the shared expert on every
 * token, with q, d the activations of x (moe_quant_act; with MOE_ACT_ROW one
 * scale per token, d [T], and one block spanning the row below):
 *   g[r] = sg[r] * sum_b d[t,b] * P_gate[r,b],  P = exact int32 block dots
 *   u[r] = su[r] * sum_b d[t,b] * P_up[r,b]
 *   h[r] = silu(g[r]) * u[r],  silu(z) = z / (1 + e^-z)
 *   (q_h, d_h) = Q8_0(h)
 *   y[j] = sd[j] * sum_b d_h[b] * P_down[j,b]
 * expert_out [T][K][H] receives y of slot (t, k) (unweighted; rows of
 * slots with idx -1 are not written);
 * shared_out [T][H] receives the shared expert's y (required iff n_shared).
 * Grouping (moe_group) runs inside this call on idx, so every distinct
 * expert's weights are streamed once for all its tokens.
 * experts: E records (see layout above); shared: one record or NULL.
 * Errors: MOE_EINVAL, MOE_EALIGN, MOE_EWORKSPACE, MOE_EHIP.
 * ------------------------------------------------------------------------- */
size_t moe_expert_ffn_workspace(const moe_cfg *cfg, int32_t T);
int moe_expert_ffn(const moe_cfg *cfg, int32_t T, const int8_t *q, const float *d,
                   const int32_t *idx, const void *experts, const void *shared,
                   float *expert_out, float *shared_out, void *workspace, size_t ws_bytes,
                   const moe_ffn_debug *dbg, void *stream);

/* ---------------------------------------------------------------------------
 * moe_combine — weighted sum of the routed experts plus the shared expert
 * ("Show HN…", 実装済みの主な機能, router item: routed_scaling_factor and
 * shared expert):
 *   y[t] = residual[t] + shared_out[t] + sum_k w[t,k] * expert_out[t,k]
 * residual and shared_out may be NULL (treated as 0).  A term with
 * w[t,k] == 0 is skipped and its expert_out row not read (top-p drops).  If y_norm is not NULL
 * it receives y[t] / sqrt(mean(y[t]^2) + eps) (unit-gain RMSNorm, the input
 * of the next layer in a pre-norm stack); y_norm must not overlap y.  y may
 * be residual itself (each element is read before it is written).
 * Errors: MOE_EINVAL (also for overlapping y and y_norm), MOE_EALIGN.
 * ------------------------------------------------------------------------- */
int moe_combine(int32_t T, int32_t H, int32_t K, const float *expert_out, const float *w,
                const float *shared_out, const float *residual, float *y, float *y_norm,
                float eps, void *stream);

/* Unit-gain RMSNorm of T rows of H floats: y = x / sqrt(mean(x^2) + eps);
 * y must not overlap x (MOE_EINVAL). */
int moe_rmsnorm(int32_t T, int32_t H, const float *x, float *y, float eps, void *stream);

/* Optional kernel timestamps for moe_layer (pass NULL in production).  For
 * each stage whose start/stop are not NULL (hipEvent_t created by the
 * caller on the device of `stream`), the stage's kernel is launched with
 * hipExtLaunchKernelGGL so that the two events carry the kernel's own
 * dispatch start and completion times; hipEventElapsedTime(start, stop)
 * is then that kernel's duration.  No extra work is enqueued. */
enum {
  MOE_STAGE_ROUTER_SCORES = 0,
  MOE_STAGE_ROUTER_SELECT = 1,
  MOE_STAGE_QUANT = 2,
  MOE_STAGE_GROUP = 3,
  MOE_STAGE_GATE_UP = 4,
  MOE_STAGE_DOWN = 5,
  MOE_STAGE_COMBINE = 6,
  MOE_STAGE_NORM = 7,
  MOE_N_STAGES = 8
};
typedef struct moe_events {
  void *start[MOE_N_STAGES];
  void *stop[MOE_N_STAGES];
} moe_events;

/* Optional device buffers moe_layer / moe_layer_ptrs fill with the step's
 * intermediates, for tests that check the integer work bit for bit (pass
 * NULL in production).  They are written by the kernels that compute the
 * step, as they compute it (for 1..16 tokens a build of the same kernels
 * with these stores added; the result y is bit-identical to a call without
 * dumps).  Any member may be NULL, except that the six union arrays are
 * given together or not at all.
 *   q, d        int8 [T][H], fp32 [T][H/32]   Q8_0 of x ("Show HN…",
 *               実装済みの主な機能, integer-dot item)
 *   counts .. n_active   the batch union in moe_group's format ("Show
 *               HN…", 実装済みの主な機能, batch-union item): the experts the
 *               step reads, each once, and the (token, rank) slots of each
 *   ffn         as for moe_expert_ffn: gate/up/down block dots, h, Q8_0 of h
 *               (pair p < T*K = slot p, pair T*K + t = the shared expert on
 *               token t). */
typedef struct moe_layer_debug {
  int8_t *q;
  float *d;
  int32_t *counts, *offsets, *perm, *inv, *active, *n_active;
  moe_ffn_debug ffn;
} moe_layer_debug;

/* ---------------------------------------------------------------------------
 * moe_layer — the whole step: routing, Q8_0 of x, grouping, expert FFNs and
 * combine on one stream, with all intermediates in the workspace.  For 1..16
 * tokens (FP8 experts: 1..4; with T*top_k <= 256) it runs as four kernels:
 * router scores (MOE_STAGE_ROUTER_SCORES); per-token selection beside the shared expert's
 * gate/up (MOE_STAGE_ROUTER_SELECT); batch union and routed gate/up with the
 * Q8_0 of h (MOE_STAGE_GATE_UP); down with the combine (MOE_STAGE_DOWN);
 * then, when y_norm is given, the RMSNorm (MOE_STAGE_NORM).  Otherwise it
 * chains the kernels of moe_route, moe_quant_act, moe_expert_ffn and
 * moe_combine (MOE_STAGE_COMBINE, which includes the RMSNorm).  Both give the same
 * arithmetic as the separate calls (bit-identical idx and int32 block dots;
 * float outputs within rounding of the summation order).
 * Workspace: any contents on entry (every byte a call reads was written
 * earlier in the same call); calls that overlap on the same workspace race.
 * x [T][H] is the (already normalised) layer input; y [T][H] the output
 * (plus residual when given); y_norm optional as in moe_combine.  idx_out and
 * w_out ([T][K], nullable) receive the routing decision.  ev: optional
 * kernel timestamps (see moe_events), dbg: optional dumps (see
 * moe_layer_debug); both NULL in production.
 * Errors: as the calls it makes.
 * ------------------------------------------------------------------------- */
size_t moe_layer_workspace(const moe_cfg *cfg, int32_t T);
int moe_layer(const moe_cfg *cfg, int32_t T, const float *x, const float *w_router,
              const float *bias, const void *experts, const void *shared,
              const float *residual, float *y, float *y_norm, float eps, int32_t *idx_out,
              float *w_out, void *workspace, size_t ws_bytes, const moe_events *ev,
              const moe_layer_debug *dbg, void *stream);

/* ---------------------------------------------------------------------------
 * moe_layer_ptrs — moe_layer with the routed expert records addressed one by
 * one: expert_ptrs is a device array of E pointers, entry e the record of
 * routed expert e (layout as above, 256-byte aligned), in any memory the
 * device can read — HBM, or pinned host memory for experts not resident on
 * the GPU (read over the host link as the kernels stream them).  This is
 * the device side of an expert cache for models larger than HBM ("Show
 * HN…", section ディスクストリーミングベースの MoE 実行方式: experts streamed
 * on demand into a cache, the learning cache pinning frequent ones): a
 * caller can move records between host and HBM and rewrite table entries
 * between calls (see moe_cache_*).  Same results as moe_layer on the same
 * record bytes; same arguments, workspace and errors otherwise.
 * ------------------------------------------------------------------------- */
int moe_layer_ptrs(const moe_cfg *cfg, int32_t T, const float *x, const float *w_router,
                   const float *bias, const void *const *expert_ptrs, const void *shared,
                   const float *residual, float *y, float *y_norm, float eps, int32_t *idx_out,
                   float *w_out, void *workspace, size_t ws_bytes, const moe_events *ev,
                   const moe_layer_debug *dbg, void *stream);

/* ---------------------------------------------------------------------------
 * moe_layer_noalloc — moe_layer for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the workspace is a static device array inside the
 * library, MOE_NOALLOC_SCRATCH_BYTES per device, held by each device that
 * runs the library until the process ends; the call itself allocates
 * nothing.  Same arguments as moe_layer without the workspace (and without
 * debug dumps), same results bit for bit.  Every call on one device shares
 * that device's array: calls that overlap on one device (two streams, two
 * threads) race.  The first call on a device also looks up the array's
 * device address there (once per device).
 * Errors: as moe_layer; MOE_EWORKSPACE when moe_layer_workspace(cfg, T)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES (at the real shape, T <= 96 fits).
 * ------------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_layer_noalloc(const moe_cfg *cfg, int32_t T, const float *x, const float *w_router,
                      const float *bias, const void *experts, const void *shared,
                      const float *residual, float *y, float *y_norm, float eps,
                      int32_t *idx_out, float *w_out, const moe_events *ev, void *stream);

/* ---------------------------------------------------------------------------
 * Expert cache (host runtime around moe_layer_ptrs) — "Show HN…", section
 * ディスクストリーミングベースの MoE 実行方式 (per-layer LRU cache and pinned hot
 * store for experts loaded on demand) and section Learning cache (usage of
 * routed experts recorded, the hottest pinned at start-up).  One cache per
 * layer.  The cold copy of every routed record is in pinned host memory
 * (host_records[e]: device-readable addresses, see moe_host_device_ptr);
 * `slots` holds n_slots records in HBM; `table` is the device array of E
 * record pointers that moe_layer_ptrs reads.  Slots [0, n_pinned) take the
 * experts with the largest counts in `usage` (nullable; ties to the lower
 * id, zero counts not pinned), copied at creation; the other slots are LRU.
 *
 * moe_cache_step is called after each moe_layer_ptrs call on the same
 * stream, with that call's idx (device, n = T*K entries, -1 allowed).  It
 * enqueues a read-back of idx; for every earlier call whose idx has landed
 * (all of them, in order, when wait != 0) it counts each distinct routed
 * expert as a hit (the call read it from HBM) or a miss (from host memory),
 * adds it to the usage counts, and promotes up to max_promote missed
 * experts per call into LRU slots (an empty slot, else the least recently
 * hit).  A victim's table entry is pointed back at host memory on `stream`
 * first; the record copy then runs on the device's copy stream (one per
 * device, shared by every cache on it, created by the first cache and kept
 * until the process ends) after an event on `stream` (so no earlier kernel
 * still reads the slot), and the new
 * entry is written on `stream` once the copy has landed (at a later call, or
 * within this call when wait != 0).  `stream` never waits for a copy; with
 * wait == 0 the host waits only when 4 read-backs are outstanding (so that
 * promotions are not queued behind many layer calls).
 *
 * moe_cache_prefetch — routing one layer ahead ("Comment exécuter un réseau
 * de neurones de 744 milliards de paramètres…", section "Comment fonctionne
 * le moteur", step 1: the next layer is routed early on a prefetch thread, a
 * prediction right about 71 % of the time, so that expert reads overlap
 * compute).  idx (device, n <= max_pairs entries, -1 skipped) is a predicted
 * routing of this cache's layer, typically moe_route with this layer's
 * router and bias on the previous layer's input, enqueued before the
 * previous layer.  The call reads idx back (the host waits for `stream` to
 * reach it), then starts promotions of the predicted experts that are
 * neither resident nor being copied, at most max_promote, into LRU victims
 * exactly as moe_cache_step does (predicted experts already resident are
 * marked used first, so the prefetch does not evict them), and returns: the
 * copies run on the copy stream while the caller enqueues the previous
 * layer.  No hit, miss or usage counts change (the call has not happened);
 * stats.prefetched counts the promotions it started.
 * moe_cache_publish, called just before this layer's moe_layer_ptrs on the
 * same stream, makes `stream` wait for every copy of this cache still in
 * flight and then points their table entries at the slots (on `stream`), so
 * the call reads them from HBM and counts them as hits.  Without it, copies
 * are published by moe_cache_step once the host sees them landed, and
 * `stream` never waits.
 * Results of moe_layer_ptrs do not depend on the cache state (same bytes
 * either way).  A cache is not thread-safe (caches used from different
 * threads are independent); not capturable in a HIP graph.  create
 * allocates host memory (the handle, a pinned read-back ring); destroy waits
 * for this cache's copies and frees them (create also allocates a pinned
 * buffer of max_pairs entries for predictions).
 * Errors: MOE_EINVAL, MOE_EALIGN (slots 256-byte, table 8-byte, every host
 * record 256-byte aligned), MOE_EHIP.
 * ------------------------------------------------------------------------- */
typedef struct moe_cache moe_cache;
typedef struct moe_cache_stats {
  uint64_t steps;        /* calls accounted (idx landed) */
  uint64_t routed;       /* distinct routed experts over those calls */
  uint64_t hits;         /* of which read from HBM */
  uint64_t misses;       /* of which read from host memory */
  uint64_t promotions;   /* record copies started */
  uint64_t completed;    /* record copies landed and published */
  uint64_t bytes_copied; /* host -> HBM bytes of the promotions */
  int32_t resident;      /* experts whose entry points at HBM now */
  uint64_t prefetched;   /* of the promotions, those moe_cache_prefetch started */
} moe_cache_stats;

/* Device-readable address of pinned host memory (hipHostGetDevicePointer). */
int moe_host_device_ptr(const void *host, void **dev);
int moe_cache_create(const moe_cfg *cfg, int32_t n_slots, int32_t n_pinned, int32_t max_promote,
                     int32_t max_pairs, const void *const *host_records, void *slots,
                     void *table, const uint64_t *usage, void *stream, moe_cache **out);
int moe_cache_step(moe_cache *c, const int32_t *idx, int32_t n, int32_t wait, void *stream);
int moe_cache_prefetch(moe_cache *c, const int32_t *idx, int32_t n, void *stream);
int moe_cache_publish(moe_cache *c, void *stream);
int moe_cache_get_stats(const moe_cache *c, moe_cache_stats *s);
/* usage [E]: the recorded counts (start-up counts included), for the next
 * run's pinning; slot_of [E]: slot of each expert, -1 when read from host. */
int moe_cache_usage(const moe_cache *c, uint64_t *usage);
int moe_cache_slot_of(const moe_cache *c, int32_t *slot_of);
int moe_cache_destroy(moe_cache *c);
/* The cache policy alone on the host, for tests: n_steps calls of n idx
 * entries each, copies landing before the next call (as with wait != 0);
 * pred (nullable, [n_steps][n]): a prediction prefetched before each call,
 * its copies landed before the call; hits/misses per call [n_steps], final
 * slot_of [n_experts]. */
int moe_cache_simulate(int32_t n_experts, int32_t n_slots, int32_t n_pinned, int32_t max_promote,
                       const uint64_t *usage, const int32_t *idx, const int32_t *pred,
                       int32_t n_steps, int32_t n, int32_t *hits, int32_t *misses,
                       int32_t *slot_of);

/* ---------------------------------------------------------------------------
 * moe_mfma_peak — measurement helper, not part of the layer: n_wg workgroups
 * of 4 waves, each wave running iters x 8 independent int8 MFMAs
 * (v_mfma_i32_16x16x64_i8, 32768 operations each) and nothing else, so that
 * n_wg * 4 * iters * 8 * 32768 int8 operations divided by the launch's time
 * is the matrix-core rate the chip reaches in practice.  out [n_wg * 256]
 * int32 (device, caller-owned) receives a checksum per thread so that no
 * work is elided.  Errors: MOE_EINVAL for n_wg outside [1, 2^20], iters
 * outside [1, 2^21) or a NULL out.
 */
int moe_mfma_peak(int32_t n_wg, int32_t iters, int32_t *out, void *stream);

/* ---------------------------------------------------------------------------
 * moe_read_peak — measurement helper, not part of the layer: n_wg
 * workgroups of 256 threads read buf [bytes] (device, 16-byte aligned,
 * bytes a positive multiple of 16) once, 16 bytes per load with the expert
 * kernels' non-temporal loads, four in flight per thread, grid-stride, so
 * that bytes divided by the launch's time is the HBM read rate the chip
 * reaches for that many bytes.  out [n_wg * 4] uint32 (device,
 * caller-owned) receives the XOR of every 32-bit word each wave read (their
 * XOR over all of out is the XOR of the whole buffer).  ev_start / ev_stop:
 * optional hipEvent_t handles (NULL: none) stamped by the kernel's own
 * dispatch, as moe_events are for the layer's stages.  Errors: MOE_EINVAL
 * for bytes not a positive multiple of 16, n_wg outside [1, 2^20], or a
 * NULL buf or out; MOE_EALIGN for a buf or out not 16-byte aligned.
 */
int moe_read_peak(const void *buf, int64_t bytes, int32_t n_wg, uint32_t *out, void *ev_start,
                  void *ev_stop, void *stream);

/* Name of a return code, and the calling thread's last detailed message. */
const char *moe_strerror(int code);
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */

// The whole routed-MoE layer step for small batches (1..16 tokens) as ONE
// kernel launch with ordered, dependency-counted work items.
//
// Same method and arithmetic as the separate calls (router: "Show HN: 遅い
// コンピュータで GLM 5.2 を実行する", 実装済みの主な機能, router item; Q8_0
// activations and the int4/int2 integer-dot kernels: same list; batch union:
// same list and "Comment exécuter un réseau de neurones de 744 milliards de
// paramètres…", "Comment fonctionne le moteur").  Why one kernel: a decode
// step streams ~177 MB (~22 us at 8 TB/s) but is a chain of dependent stages;
// as separate launches each stage pays ~4-6 us of launch and ramp latency.
// Here the stages overlap: the shared expert streams while the router runs,
// and each expert's down projection starts as soon as its h is complete.
//
// Workgroup roles, in blockIdx order (a workgroup only ever waits for work
// done by workgroups with a lower index, so in-order dispatch cannot
// deadlock; every wait is bounded and records a timeout in the error word):
//   [0, n_router)        router items, two experts each: Q8_0 of a slice of
//                        x, fixed-order fp32 logits, sigmoid; the last one
//                        to finish selects the experts of every token and
//                        groups the slots (batch union), then raises READY.
//   [.., + nw_gu)        gate/up workers: items (expert slot, 32-row block
//                        of h), slot-major with the shared expert first;
//                        each item computes h = silu(gate)*up for 32 rows and
//                        writes its Q8_0 block, then counts HDONE[slot].
//   [.., + nw_dn)        down workers: items (expert slot, 32-row tile of
//                        the output); weights are loaded before waiting for
//                        HDONE[slot]; the last slot to finish a tile combines
//                        it (y = residual + shared + sum_k w_k expert_k, in
//                        rank order) and, with y_norm, the last tile applies
//                        the unit-gain RMSNorm to whole rows.
// Counters live in a zero-initialised region of the workspace, one per
// 256-byte line (same-address atomics serialise); every call returns them to
// zero: tile and route counters are cleared by their last user, the rest by
// the last workgroup to exit (a 64-way tree of exit counters).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace lf {

constexpr int TMAX = 16;   // tokens per call on this path
constexpr int NSUB = 64;   // exit sub-counters
constexpr int LINE = 64;   // uint32 words per counter line (256 B)
constexpr int MAX_SLOTS = 272;
constexpr int MAX_TILES = 256;
// counter word indices (times LINE)
constexpr int C_ROUTE = 1, C_READY = 2, C_TOP = 3, C_NORM = 4, C_ERR = 5;
constexpr int C_RSUB = 8;   // 16 router sub-counters
constexpr int C_EXIT = C_RSUB + 16;
constexpr int C_HDONE = C_EXIT + NSUB;
constexpr int C_TILE = C_HDONE + MAX_SLOTS;
constexpr int C_END = C_TILE + MAX_TILES;
constexpr uint32_t SPIN_MAX = 1u << 20;  // ~1 s: each poll is a memory round trip

}  // namespace lf

size_t layer_fused_sync_bytes() { return (size_t)lf::C_END * lf::LINE * sizeof(uint32_t); }

__device__ __forceinline__ uint32_t *ctr(const LayerArgs &a, int c) { return a.sync + (size_t)c * lf::LINE; }

__device__ __forceinline__ void release_fence() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ uint32_t atomic_add_relaxed(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_relaxed(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_rel(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
// Every wave's outstanding global stores complete (a wait, no cache action).
__device__ __forceinline__ void drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cache maintenance is per CU (L1) and per XCD (L2), not per thread: an
// agent-scope acquire invalidates, a release writes back.  So one thread
// per block performs them, bracketed by block barriers, and polling uses
// relaxed loads (an acquire per poll would invalidate the L2 the streaming
// workgroups depend on).

// Thread 0 waits (bounded) until *p >= v, then acquires for the block.
// Must be called by every thread of the block.
__device__ void block_wait_geq(const LayerArgs &a, const uint32_t *p, uint32_t v) {
  if (threadIdx.x == 0) {
    uint32_t n = 0;
    while (atomic_load_relaxed(p) < v) {
      __builtin_amdgcn_s_sleep(2);
      if (++n >= lf::SPIN_MAX) {
        atomic_add_relaxed(ctr(a, lf::C_ERR), 1u);
        break;
      }
    }
    acquire_fence();
  }
  __syncthreads();
}

// All threads: the block's global writes are made visible device-wide, then
// thread 0 adds 1 to *p; the old value is broadcast to the block.  A block
// that finds itself last (and will read what the others wrote) must call
// block_acquire() first.
__device__ uint32_t block_signal(uint32_t *p, uint32_t *lds_word) {
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    release_fence();
    *lds_word = atomic_add_relaxed(p, 1u);
  }
  __syncthreads();
  const uint32_t old = *lds_word;
  __syncthreads();
  return old;
}

__device__ void block_acquire() {
  if (threadIdx.x == 0) acquire_fence();
  __syncthreads();
}

__device__ __forceinline__ void stamp(const LayerArgs &a, int k) {
  if (a.trace && threadIdx.x == 0 && (uint64_t)(blockIdx.x * 4 + 4) <= a.trace_words)
    a.trace[(size_t)blockIdx.x * 4 + k] = wall_clock64();
}

// Q8_0 of the x rows a worker is using, cached in LDS: xq_tok[i] = token
// held in row i (-1 = none); valid for gate/up items only.
constexpr int XQ_ROWS = 4;  // rows of the dynamic LDS cache (fewer when T < 4)

struct LfShared {
  uint32_t word;
  int n_active;
  int ready;
  int pad;
  int xq_tok[XQ_ROWS];
  union {
    float part[2][lf::TMAX][128];  // router chunk partials
    struct {
      float sb[lf::TMAX * 256];    // selection: biased scores (T*E <= 4096)
      int32_t idx[256];
      float wv[256];
      int32_t cnt[1024];
      int32_t off[1025];
      int32_t wt[16];
    } fin;
    float hb[4][32];               // gate/up: h of one 32-row block, up to 4 tokens
    float red[16][4];              // combine: per-token partial sums of squares
  } u;
};

// ------------------------------------------------------------ router items

__device__ __forceinline__ float exp_fixed_lf(float y) {
  y = y > 87.0f ? 87.0f : y;
  y = y < -87.0f ? -87.0f : y;
  const float n = __builtin_rintf(y * 1.44269502f);
  float r = __builtin_fmaf(-n, 0.693145751953125f, y);
  r = __builtin_fmaf(-n, 1.42860677e-06f, r);
  float p = 1.98412701e-04f;
  p = __builtin_fmaf(p, r, 1.38888892e-03f);
  p = __builtin_fmaf(p, r, 8.33333377e-03f);
  p = __builtin_fmaf(p, r, 4.16666679e-02f);
  p = __builtin_fmaf(p, r, 1.66666672e-01f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)n);
}

// Q8_0 of one 32-block with 8 lanes x 4 values (lanes of a block are
// consecutive and all active); returns the packed 4 codes, d via *dd.
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

// Selection of one token by one wave, scores of the token in LDS (sb) and
// global (s).  Same rule as k_router_select.
__device__ void select_token_wave(const LayerArgs &a, LfShared &sm, int t) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, G = a.G, gs = E / G;
  const float *sb = sm.u.fin.sb + t * E;
  float gscore = -INFINITY;
  if (lane < G) {
    float m1 = -INFINITY, m2 = -INFINITY;
    for (int e = lane * gs; e < (lane + 1) * gs; e++) {
      const float v = sb[e];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    gscore = m1 + m2;
  }
  bool kept = false;
  for (int j = 0; j < a.TG; j++) {
    unsigned long long key = 0;
    if (lane < G && !kept)
      key = ((unsigned long long)float_key(gscore) << 32) | (0xFFFFFFFFu - (uint32_t)lane);
    key = wave_max_u64(key);
    int g = (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
    g = (g >= 0 && g < G) ? g : 0;
    if (lane == g) kept = true;
  }
  const unsigned long long kept_mask = __ballot(kept);
  uint32_t taken = 0;
  int my_e = -1;  // lane k < K: the k-th selection
  for (int k = 0; k < a.K; k++) {
    unsigned long long best = 0;
    for (int j = 0; j * 64 + lane < E; j++) {
      const int e = j * 64 + lane;
      if (((kept_mask >> (e / gs)) & 1ull) && !((taken >> j) & 1u)) {
        const unsigned long long key =
            ((unsigned long long)float_key(sb[e]) << 32) | (0xFFFFFFFFu - (uint32_t)e);
        best = key > best ? key : best;
      }
    }
    best = wave_max_u64(best);
    int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    e = (e >= 0 && e < E) ? e : 0;
    if ((e & 63) == lane) taken |= 1u << (e >> 6);
    if (lane == k) my_e = e;
  }
  // unbiased scores of the selections, summed in rank order
  const float sv = (lane < a.K) ? a.s[(size_t)t * E + my_e] : 0.0f;
  float S = __shfl(sv, 0, 64);
  for (int k = 1; k < a.K; k++) S = S + __shfl(sv, k, 64);
  if (lane < a.K) {
    const float wk = (sv / S) * a.scale;
    a.idx[t * a.K + lane] = my_e;
    a.w[t * a.K + lane] = wk;
    sm.u.fin.idx[t * a.K + lane] = my_e;
    sm.u.fin.wv[t * a.K + lane] = wk;
  }
}

// Block-wide exclusive scan of one value per thread (256 threads).
__device__ int block_exscan256(int v, int *wt, int *total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wt[wv] = x;
  __syncthreads();
  int pre = 0, all = 0;
  for (int w = 0; w < 4; w++) {
    pre += (w < wv) ? wt[w] : 0;
    all += wt[w];
  }
  __syncthreads();
  *total = all;
  return pre + x - v;
}

// The last router item: select every token, then group the T*K slots.
__device__ void finish_route(const LayerArgs &a, LfShared &sm) {
  const int E = a.E, T = a.T, K = a.K, n = T * K;
  for (int i = threadIdx.x; i < T * E; i += 256) sm.u.fin.sb[i] = a.sb[i];
  __syncthreads();
  for (int t = threadIdx.x >> 6; t < T; t += 4) select_token_wave(a, sm, t);
  for (int e = threadIdx.x; e < E; e += 256) sm.u.fin.cnt[e] = 0;
  __syncthreads();
  if (threadIdx.x < n) atomicAdd(&sm.u.fin.cnt[sm.u.fin.idx[threadIdx.x]], 1);
  __syncthreads();
  // exclusive scan over experts: thread i owns experts [4i, 4i+4)
  int c[4], loc = 0, act = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = threadIdx.x * 4 + j;
    c[j] = e < E ? sm.u.fin.cnt[e] : 0;
    loc += c[j];
    act += c[j] > 0;
  }
  int n_used, n_act;
  int pre = block_exscan256(loc, sm.u.fin.wt, &n_used);
  int apre = block_exscan256(act, sm.u.fin.wt + 4, &n_act);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = threadIdx.x * 4 + j;
    if (e < E) {
      sm.u.fin.off[e] = pre;
      a.offsets[e] = pre;
      a.counts[e] = c[j];
      a.active[e] = -1;
    }
    pre += c[j];
  }
  if (threadIdx.x == 0) {
    sm.u.fin.off[E] = n_used;
    a.offsets[E] = n_used;
    a.n_active[0] = n_act;
  }
  __syncthreads();  // active[] = -1 before the compaction
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = threadIdx.x * 4 + j;
    if (e < E && c[j] > 0) a.active[apre++] = e;
  }
  if (threadIdx.x < n) {
    const int s = threadIdx.x, e = sm.u.fin.idx[s];
    int rank = 0;
    for (int j = 0; j < s; j++) rank += sm.u.fin.idx[j] == e;
    a.perm[sm.u.fin.off[e] + rank] = s;
  }
}

// Router item r: logits of experts 2r and 2r+1 for every token (thread l <
// H/64 of each half owns chunk l: an fma chain over 64 elements; the chunk
// partials are added left to right by one thread per token), sigmoid, bias.
// The last item to finish selects and groups, then raises READY.
__device__ void router_item(const LayerArgs &a, LfShared &sm, int r) {
  const int tid = threadIdx.x;
  const int H = a.H, E = a.E, T = a.T;
  const int half = tid >> 7, l = tid & 127;
  const int e = 2 * r + half;
  const int nch = H / 64;
  if (e < E && l < nch) {
    const float4 *w4 = reinterpret_cast<const float4 *>(a.wr + (size_t)e * H + l * 64);
    float4 wv[16];
#pragma unroll
    for (int k = 0; k < 16; k++) wv[k] = w4[k];
    for (int t = 0; t < T; t++) {
      const float4 *x4 = reinterpret_cast<const float4 *>(a.x + (size_t)t * H + l * 64);
      float acc = 0.0f;
#pragma unroll
      for (int h2 = 0; h2 < 2; h2++) {  // the chain runs in index order over both halves
        float4 xv[8];
#pragma unroll
        for (int k = 0; k < 8; k++) xv[k] = x4[8 * h2 + k];
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const float4 wk = wv[8 * h2 + k];
          acc = __builtin_fmaf(xv[k].x, wk.x, acc);
          acc = __builtin_fmaf(xv[k].y, wk.y, acc);
          acc = __builtin_fmaf(xv[k].z, wk.z, acc);
          acc = __builtin_fmaf(xv[k].w, wk.w, acc);
        }
      }
      sm.u.part[half][t][l] = acc;
    }
  }
  __syncthreads();
  if (e < E && l < T) {
    float tot = sm.u.part[half][l][0];
    for (int c = 1; c < nch; c++) tot = tot + sm.u.part[half][l][c];
    const float sv = 1.0f / (1.0f + exp_fixed_lf(-tot));
    a.s[(size_t)l * E + e] = sv;
    a.sb[(size_t)l * E + e] = sv + a.bias[e];
  }
  // two-level count (same-address atomics serialise): 16 sub-counters
  const int sub = r % 16;
  const uint32_t in_sub = (uint32_t)((a.n_router - 1 - sub) / 16 + 1);
  uint32_t old = block_signal(ctr(a, lf::C_RSUB + sub), &sm.word);
  if (old != in_sub - 1) return;
  const uint32_t subs = (uint32_t)(a.n_router < 16 ? a.n_router : 16);
  old = block_signal(ctr(a, lf::C_ROUTE), &sm.word);
  if (old != subs - 1) return;
  block_acquire();
  finish_route(a, sm);
  drain_stores();
  __syncthreads();
  if (tid == 0) {
    for (int i = 0; i < 16; i++) *ctr(a, lf::C_RSUB + i) = 0u;  // every item has counted
    *ctr(a, lf::C_ROUTE) = 0u;
    atomic_store_rel(ctr(a, lf::C_READY), 1u);
  }
}

// ------------------------------------------------------------ expert slots

struct Slot {
  const uint8_t *blob;
  int n_tok;
  bool shared;
  const int32_t *list;
};

__device__ __forceinline__ Slot slot_of(const LayerArgs &a, int slot) {
  Slot s;
  if (slot < a.n_shared) {
    s.blob = a.shared;
    s.n_tok = a.T;
    s.shared = true;
    s.list = nullptr;
  } else {
    // indices read from device memory are clamped so that a timed-out wait
    // can only produce wrong values, never an out-of-bounds access
    const int n_slots = a.T * a.K;
    int e = a.active[slot - a.n_shared];
    e = min(max(e, 0), a.E - 1);
    const int lo = min(max(a.offsets[e], 0), n_slots);
    const int hi = min(max(a.offsets[e + 1], lo), n_slots);
    s.blob = a.experts + (size_t)e * a.blob_bytes;
    s.n_tok = hi - lo;
    s.shared = false;
    s.list = a.perm + lo;
  }
  return s;
}

__device__ __forceinline__ void tok_pair(const LayerArgs &a, const Slot &s, int i, int &tok,
                                         int &pair) {
  if (s.shared) {
    tok = i;
    pair = a.T * a.K + i;
  } else {
    const int sl = min(max(s.list[i], 0), a.T * a.K - 1);
    tok = sl / a.K;
    pair = sl;
  }
}

__device__ __forceinline__ float silu_lf(float z) { return z / (1.0f + __expf(-z)); }

// Activation operand of one weight piece for one token.
template <int WB>
struct Act;
template <>
struct Act<4> {
  QBlock q;
  float d;  // d / 16
};
template <>
struct Act<2> {
  int f[4][4];
  float da, db;  // d / 64 of the two blocks of the piece
};

template <int WB>
__device__ __forceinline__ void load_act(const int8_t *q, const float *d, int p, bool ok,
                                         Act<WB> &o);
template <>
__device__ __forceinline__ void load_act<4>(const int8_t *q, const float *d, int p, bool ok,
                                            Act<4> &o) {
  uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
  float dd = 0.0f;
  if (ok) {
    const uint4 *qp = reinterpret_cast<const uint4 *>(q + 32 * p);
    x0 = qp[0];
    x1 = qp[1];
    dd = d[p] * (1.0f / 16.0f);
  }
  o.q = split_block(x0, x1);
  o.d = dd;
}
template <>
__device__ __forceinline__ void load_act<2>(const int8_t *q, const float *d, int p, bool ok,
                                            Act<2> &o) {
  uint4 z[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                make_uint4(0, 0, 0, 0)};
  float d0 = 0.0f, d1 = 0.0f;
  if (ok) {
    const uint4 *qp = reinterpret_cast<const uint4 *>(q + 64 * p);
#pragma unroll
    for (int j = 0; j < 4; j++) z[j] = qp[j];
    d0 = d[2 * p] * (1.0f / 64.0f);
    d1 = d[2 * p + 1] * (1.0f / 64.0f);
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
#pragma unroll
    for (int fi = 0; fi < 4; fi++) {
      const uint32_t sel = (uint32_t)(fi | ((4 + fi) << 8)) | 0x0C0C0000u;
      const uint32_t a01 = __builtin_amdgcn_perm(z[j].y, z[j].x, sel);
      const uint32_t a23 = __builtin_amdgcn_perm(z[j].w, z[j].z, sel);
      o.f[fi][j] = (int)__builtin_amdgcn_perm(a23, a01, 0x05040100u);
    }
  }
  o.da = d0;
  o.db = d1;
}

// fp32 contribution of one weight piece against one token: sum_b d_b * P_b.
template <int WB>
__device__ __forceinline__ float piece_dot(const uint4 w, const Act<WB> &a);
template <>
__device__ __forceinline__ float piece_dot<4>(const uint4 w, const Act<4> &a) {
  return (float)dot_int4_block16(w, a.q) * a.d;
}
template <>
__device__ __forceinline__ float piece_dot<2>(const uint4 w, const Act<2> &a) {
  int x = 0, y = 0;
#pragma unroll
  for (int fi = 0; fi < 4; fi++) {
    x = sdot4(int2_field64(w.x, fi), a.f[fi][0], x);
    x = sdot4(int2_field64(w.y, fi), a.f[fi][1], x);
    y = sdot4(int2_field64(w.z, fi), a.f[fi][2], y);
    y = sdot4(int2_field64(w.w, fi), a.f[fi][3], y);
  }
  return fmaf((float)x, a.da, (float)y * a.db);
}

// Q8_0 of the activation block(s) under one weight piece, computed by the
// lane itself from x (same rule and fp32 steps as moe_quant_act: amax, d =
// amax/127, q = roundf(x * (1/d)) clamped), already in the operand layout.
__device__ __forceinline__ uint32_t q8_code(float f, float id) {
  float r = roundf(f * id);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (uint32_t)(uint8_t)(int8_t)(int)r;
}
__device__ __forceinline__ float q8_scale(const float *v, int n, float *id) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < n; i++) m = fmaxf(m, fabsf(v[i]));
  const float dd = m / 127.0f;
  *id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
  return dd;
}

template <int WB>
__device__ __forceinline__ void act_from_x(const float *xt, int p, bool ok, Act<WB> &o);
template <>
__device__ __forceinline__ void act_from_x<4>(const float *xt, int p, bool ok, Act<4> &o) {
  float v[32];
  const float4 *x4 = reinterpret_cast<const float4 *>(xt + 32 * p);
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const float4 f = ok ? x4[k] : make_float4(0.f, 0.f, 0.f, 0.f);
    v[4 * k] = f.x;
    v[4 * k + 1] = f.y;
    v[4 * k + 2] = f.z;
    v[4 * k + 3] = f.w;
  }
  float id;
  const float dd = q8_scale(v, 32, &id);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    o.q.ev[j] = (int)(q8_code(v[8 * j], id) | (q8_code(v[8 * j + 2], id) << 8) |
                      (q8_code(v[8 * j + 4], id) << 16) | (q8_code(v[8 * j + 6], id) << 24));
    o.q.od[j] = (int)(q8_code(v[8 * j + 1], id) | (q8_code(v[8 * j + 3], id) << 8) |
                      (q8_code(v[8 * j + 5], id) << 16) | (q8_code(v[8 * j + 7], id) << 24));
  }
  o.d = dd * (1.0f / 16.0f);
}
template <>
__device__ __forceinline__ void act_from_x<2>(const float *xt, int p, bool ok, Act<2> &o) {
  float v[64];
  const float4 *x4 = reinterpret_cast<const float4 *>(xt + 64 * p);
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const float4 f = ok ? x4[k] : make_float4(0.f, 0.f, 0.f, 0.f);
    v[4 * k] = f.x;
    v[4 * k + 1] = f.y;
    v[4 * k + 2] = f.z;
    v[4 * k + 3] = f.w;
  }
  float id0, id1;
  const float d0 = q8_scale(v, 32, &id0);
  const float d1 = q8_scale(v + 32, 32, &id1);
  // word j covers codes 16j .. 16j+15 (block 0 for j < 2); byte i of field fi
  // is the activation of code 16j + 4i + fi
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const float id = j < 2 ? id0 : id1;
#pragma unroll
    for (int fi = 0; fi < 4; fi++)
      o.f[fi][j] = (int)(q8_code(v[16 * j + fi], id) | (q8_code(v[16 * j + 4 + fi], id) << 8) |
                         (q8_code(v[16 * j + 8 + fi], id) << 16) |
                         (q8_code(v[16 * j + 12 + fi], id) << 24));
  }
  o.da = d0 * (1.0f / 64.0f);
  o.db = d1 * (1.0f / 64.0f);
}

// ------------------------------------------------------------ gate/up item

extern __shared__ uint8_t lf_dyn[];
__device__ __forceinline__ int8_t *xq_row(const LayerArgs &a, int i) {
  return reinterpret_cast<int8_t *>(lf_dyn) + (size_t)i * a.H;
}
__device__ __forceinline__ float *xd_row(const LayerArgs &a, int i) {
  return reinterpret_cast<float *>(lf_dyn + (size_t)a.xq_rows * a.H) + (size_t)i * (a.H / 32);
}

// Make LDS rows 0..n-1 hold Q8_0 of tokens toks[0..n) (row i = toks[i]);
// rows already holding the right token are kept.  Whole block.
__device__ void xq_ensure(const LayerArgs &a, LfShared &sm, const int *toks, int n) {
  bool same = true;
  for (int i = 0; i < n; i++) same = same && (sm.xq_tok[i] == toks[i]);
  if (same) return;  // uniform: every thread reads the same LDS words
  __syncthreads();
  const int H = a.H, nbt = H / 32;
  for (int v = threadIdx.x; v < n * nbt * 8; v += 256) {
    const int i = v / (nbt * 8), rem = v % (nbt * 8);
    const int blk = rem >> 3, sub = rem & 7;
    const float4 x = reinterpret_cast<const float4 *>(a.x + (size_t)toks[i] * H)[blk * 8 + sub];
    float dd;
    const uint32_t packed = q8_quad(x, &dd);
    reinterpret_cast<uint32_t *>(xq_row(a, i))[blk * 8 + sub] = packed;
    if (sub == 0) xd_row(a, i)[blk] = dd;
  }
  __syncthreads();
  if (threadIdx.x < n) sm.xq_tok[threadIdx.x] = toks[threadIdx.x];
  __syncthreads();
}

// 32 rows of h for one expert slot; wave wv owns rows 8wv .. 8wv+7, streamed
// in batches of 2 (a gate and an up row each); the activations come from the
// worker's LDS copy of Q8_0(x).
template <int WB, int TT, int NPL>
__device__ void gate_up_item(const LayerArgs &a, LfShared &sm, int slot, int blk) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I;
  const int per = 128 / WB;  // codes per 16-byte piece
  const int npieces = H / per;
  const size_t row_b = (size_t)H * WB / 8;
  const Slot s = slot_of(a, slot);
  const uint8_t *gate = s.blob;
  const uint8_t *up = s.blob + (size_t)I * row_b;
  const float *scales = reinterpret_cast<const float *>(s.blob + 3 * (size_t)I * row_b);
  const int rbase = blk * 32 + wv * 8;
  // all tokens at once when they fit the LDS cache (then it survives items)
  const bool whole = a.T <= XQ_ROWS;

  for (int c0 = 0; c0 < s.n_tok; c0 += TT) {
    uint4 wb[2][2][NPL];  // [row of batch][gate, up][piece]
    auto load_batch = [&](int bt) {
#pragma unroll
      for (int rr = 0; rr < 2; rr++) {
        const int r = rbase + bt * 2 + rr;
#pragma unroll
        for (int i = 0; i < NPL; i++) {
          const int p = lane + 64 * i;
          const bool ok = p < npieces;
          wb[rr][0][i] = ok ? reinterpret_cast<const uint4 *>(gate + (size_t)r * row_b)[p]
                            : make_uint4(0, 0, 0, 0);
          wb[rr][1][i] = ok ? reinterpret_cast<const uint4 *>(up + (size_t)r * row_b)[p]
                            : make_uint4(0, 0, 0, 0);
        }
      }
    };
    load_batch(0);
    int pair[TT], row[TT];
    int toks[XQ_ROWS];
    int nt = 0;
    if (whole) {
      for (int i = 0; i < a.T; i++) toks[i] = i;
      nt = a.T;
    }
#pragma unroll
    for (int t = 0; t < TT; t++) {
      int tok = 0;
      pair[t] = -1;
      if (c0 + t < s.n_tok) tok_pair(a, s, c0 + t, tok, pair[t]);
      if (!whole) {
        toks[t] = tok;
        nt = t + 1;
      }
      row[t] = whole ? tok : t;
    }
    xq_ensure(a, sm, toks, nt);
    Act<WB> act[NPL][TT];
#pragma unroll
    for (int t = 0; t < TT; t++) {
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        load_act<WB>(xq_row(a, row[t]), xd_row(a, row[t]), p, pair[t] >= 0 && p < npieces,
                     act[i][t]);
      }
    }
#pragma unroll
    for (int bt = 0; bt < 4; bt++) {
      if (bt > 0) load_batch(bt);
#pragma unroll
      for (int rr = 0; rr < 2; rr++) {
        const int r = rbase + bt * 2 + rr;
        float g[TT], u[TT];
#pragma unroll
        for (int t = 0; t < TT; t++) g[t] = u[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; i++) {
#pragma unroll
          for (int t = 0; t < TT; t++) {
            g[t] += piece_dot<WB>(wb[rr][0][i], act[i][t]);
            u[t] += piece_dot<WB>(wb[rr][1][i], act[i][t]);
          }
        }
        const float sg = scales[r], su = scales[I + r];
#pragma unroll
        for (int t = 0; t < TT; t++) {
          const float gv = sg * wave_sum(g[t]);
          const float uv = su * wave_sum(u[t]);
          if (lane == 0) sm.u.hb[t][wv * 8 + bt * 2 + rr] = silu_lf(gv) * uv;
        }
      }
    }
    __syncthreads();
    // Q8_0 of the 32 h values of each token: 8 lanes x 4 values per token
    if (threadIdx.x < TT * 8) {
      const int t = threadIdx.x >> 3, j = threadIdx.x & 7;
      const float4 v = make_float4(sm.u.hb[t][4 * j], sm.u.hb[t][4 * j + 1],
                                   sm.u.hb[t][4 * j + 2], sm.u.hb[t][4 * j + 3]);
      float dd;
      const uint32_t packed = q8_quad(v, &dd);
      if (pair[t] >= 0) {
        reinterpret_cast<uint32_t *>(a.qh + (size_t)pair[t] * I + blk * 32)[j] = packed;
        if (j == 0) a.dh[(size_t)pair[t] * (I / 32) + blk] = dd;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ down item

template <int WB, int TT, int NPL>
__device__ void down_item(const LayerArgs &a, LfShared &sm, int slot, int tile, int nb) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I;
  const int per = 128 / WB;
  const int npieces = I / per;
  const size_t row_b = (size_t)I * WB / 8;
  const Slot s = slot_of(a, slot);
  const uint8_t *down = s.blob + 2 * (size_t)I * ((size_t)H * WB / 8);
  const float *sd = reinterpret_cast<const float *>(s.blob + 3 * (size_t)I * ((size_t)H * WB / 8)) +
                    2 * I;
  const int j0 = tile * 32 + wv * 8;
  uint4 wd[8][NPL];
#pragma unroll
  for (int rr = 0; rr < 8; rr++) {
#pragma unroll
    for (int i = 0; i < NPL; i++) {
      const int p = lane + 64 * i;
      wd[rr][i] = (p < npieces) ? reinterpret_cast<const uint4 *>(down + (size_t)(j0 + rr) * row_b)[p]
                                : make_uint4(0, 0, 0, 0);
    }
  }
  float sdv[8];
#pragma unroll
  for (int rr = 0; rr < 8; rr++) sdv[rr] = sd[j0 + rr];
  block_wait_geq(a, ctr(a, lf::C_HDONE + slot), (uint32_t)nb);
  for (int c0 = 0; c0 < s.n_tok; c0 += TT) {
    Act<WB> act[NPL][TT];
    int pair[TT], tok[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) {
      pair[t] = -1;
      tok[t] = 0;
      if (c0 + t < s.n_tok) tok_pair(a, s, c0 + t, tok[t], pair[t]);
      const int8_t *qt = a.qh + (size_t)(pair[t] >= 0 ? pair[t] : 0) * I;
      const float *dt = a.dh + (size_t)(pair[t] >= 0 ? pair[t] : 0) * (I / 32);
#pragma unroll
      for (int i = 0; i < NPL; i++) {
        const int p = lane + 64 * i;
        load_act<WB>(qt, dt, p, pair[t] >= 0 && p < npieces, act[i][t]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 8; rr++) {
      float acc[TT];
#pragma unroll
      for (int t = 0; t < TT; t++) acc[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < NPL; i++) {
#pragma unroll
        for (int t = 0; t < TT; t++) acc[t] += piece_dot<WB>(wd[rr][i], act[i][t]);
      }
#pragma unroll
      for (int t = 0; t < TT; t++) {
        const float yv = sdv[rr] * wave_sum(acc[t]);
        if (lane == 0 && pair[t] >= 0) {
          if (s.shared)
            a.so[(size_t)tok[t] * H + j0 + rr] = yv;
          else
            a.eo[(size_t)pair[t] * H + j0 + rr] = yv;
        }
      }
    }
  }
}

// Combine of one 32-row tile for every token (and the RMSNorm bookkeeping).
__device__ void combine_tile(const LayerArgs &a, LfShared &sm, int tile, int n_tiles) {
  const int H = a.H, K = a.K, T = a.T;
  const bool norm = a.y_norm != nullptr;
  for (int base = 0; base < T * 32; base += 256) {
    const int v = base + threadIdx.x;
    const int t = v >> 5, j = tile * 32 + (v & 31);
    float acc = 0.0f;
    if (t < T) {
      if (a.residual) acc = a.residual[(size_t)t * H + j];
      if (a.n_shared) acc += a.so[(size_t)t * H + j];
      for (int k = 0; k < K; k++)
        acc = fmaf(a.w[t * K + k], a.eo[((size_t)t * K + k) * H + j], acc);
      a.y[(size_t)t * H + j] = acc;
    }
    if (norm) {
      // 32 consecutive threads hold one token's 32 rows
      float q = acc * acc;
      q += __shfl_xor(q, 1, 32);
      q += __shfl_xor(q, 2, 32);
      q += __shfl_xor(q, 4, 32);
      q += __shfl_xor(q, 8, 32);
      q += __shfl_xor(q, 16, 32);
      if ((v & 31) == 0 && t < T) a.ssq[(size_t)t * n_tiles + tile] = q;
    }
  }
  if (!norm) return;
  const uint32_t old = block_signal(ctr(a, lf::C_NORM), &sm.word);
  if (old != (uint32_t)n_tiles - 1) return;
  block_acquire();
  // last tile: whole-row RMSNorm, sums taken in tile order
  if (threadIdx.x < T) {
    float ss = 0.0f;
    for (int i = 0; i < n_tiles; i++) ss += a.ssq[(size_t)threadIdx.x * n_tiles + i];
    sm.u.red[threadIdx.x][0] = 1.0f / sqrtf(ss / (float)H + a.eps);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * (H / 4); i += 256) {
    const int t = i / (H / 4);
    float4 v = reinterpret_cast<const float4 *>(a.y)[i];
    const float inv = sm.u.red[t][0];
    v.x *= inv;
    v.y *= inv;
    v.z *= inv;
    v.w *= inv;
    reinterpret_cast<float4 *>(a.y_norm)[i] = v;
  }
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) atomic_store_rel(ctr(a, lf::C_NORM), 0u);
}

// ------------------------------------------------------------ the kernel

// Down item, its tile count, and the tile's combine when it is the last.
template <int WB, int TT, int NPD>
__device__ void down_and_combine(const LayerArgs &a, LfShared &sm, int slot, int tile) {
  const int NB = a.I / 32, NT = a.H / 32;
  down_item<WB, TT, NPD>(a, sm, slot, tile, NB);
  const uint32_t old = block_signal(ctr(a, lf::C_TILE + tile), &sm.word);
  block_wait_geq(a, ctr(a, lf::C_READY), 1u);  // n_active is known from here on
  const int n_slots = a.n_shared + min(max(a.n_active[0], 0), a.n_slots_ub - a.n_shared);
  if (old == (uint32_t)n_slots - 1) {
    block_acquire();
    combine_tile(a, sm, tile, NT);
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) atomic_store_rel(ctr(a, lf::C_TILE + tile), 0u);
  }
}

// Persistent schedule over gridDim.x co-resident workers.  A worker runs its
// items in increasing order and every item waits only for lower items, so
// the lowest unfinished item can always run.
//   stage A: router items | shared-expert gate/up | shared-expert down
//   stage B: routed gate/up (after READY), spread over all workers
//   stage C: routed down + combine
template <int WB, int TT, int NPG, int NPD>
__global__ void __launch_bounds__(256) k_layer_fused(LayerArgs a) {
  __shared__ LfShared sm;
  const int w = blockIdx.x, NW = gridDim.x;
  const int NB = a.I / 32, NT = a.H / 32;
  stamp(a, 0);
  if (threadIdx.x < XQ_ROWS) sm.xq_tok[threadIdx.x] = -1;
  __syncthreads();
  const int nr = a.n_router;
  const int nsg = a.n_shared ? NB : 0;
  const int nsd = a.n_shared ? NT : 0;
  for (int it = w; it < nr + nsg + nsd; it += NW) {
    if (it < nr) {
      router_item(a, sm, it);
    } else if (it < nr + nsg) {
      gate_up_item<WB, TT, NPG>(a, sm, 0, it - nr);
      block_signal(ctr(a, lf::C_HDONE), &sm.word);
    } else {
      down_and_combine<WB, TT, NPD>(a, sm, 0, it - nr - nsg);
    }
  }
  stamp(a, 1);
  block_wait_geq(a, ctr(a, lf::C_READY), 1u);
  const int n_act = min(max(a.n_active[0], 0), a.n_slots_ub - a.n_shared);
  for (int i = w; i < n_act * NB; i += NW) {
    const int slot = a.n_shared + i / NB;
    gate_up_item<WB, TT, NPG>(a, sm, slot, i % NB);
    block_signal(ctr(a, lf::C_HDONE + slot), &sm.word);
  }
  for (int i = w; i < n_act * NT; i += NW)
    down_and_combine<WB, TT, NPD>(a, sm, a.n_shared + i / NT, i % NT);
  stamp(a, 2);
  // exit: a 64-way tree; the very last worker clears the remaining counters
  const int sub = w % lf::NSUB;
  const uint32_t in_sub = (uint32_t)((NW - 1 - sub) / lf::NSUB + 1);
  const uint32_t old = block_signal(ctr(a, lf::C_EXIT + sub), &sm.word);
  stamp(a, 3);
  if (old != in_sub - 1) return;
  const uint32_t subs = (uint32_t)(NW < lf::NSUB ? NW : lf::NSUB);
  const uint32_t top = block_signal(ctr(a, lf::C_TOP), &sm.word);
  if (top != subs - 1) return;
  block_acquire();
  for (int i = threadIdx.x; i < a.n_slots_ub; i += 256) *ctr(a, lf::C_HDONE + i) = 0u;
  for (int i = threadIdx.x; i < lf::NSUB; i += 256) *ctr(a, lf::C_EXIT + i) = 0u;
  if (threadIdx.x == 0) {
    *ctr(a, lf::C_READY) = 0u;
    *ctr(a, lf::C_TOP) = 0u;
  }
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) release_fence();
}

bool layer_fused_supported(const moe_cfg &c, int T) {
  if (T < 1 || T > lf::TMAX) return false;
  if (T * c.n_experts > lf::TMAX * 256 || c.n_experts > 1024) return false;
  if (T * c.top_k > 256) return false;
  if (c.n_shared + (T * c.top_k < c.n_experts ? T * c.top_k : c.n_experts) > lf::MAX_SLOTS)
    return false;
  if (c.hidden / 32 > lf::MAX_TILES || c.hidden / 64 > 128) return false;
  const int per = c.wbits == 4 ? 32 : 64;
  return c.hidden / per <= 256 && c.inter / per <= 128;
}

// Workers = co-resident workgroups (occupancy x CUs), computed once per
// kernel instance and device; the schedule needs every worker resident.
template <int WB, int TT, int NPG, int NPD>
static void launch_lf(LayerArgs a, hipStream_t st, Ev ev) {
  static int workers[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (workers[dev] == 0) {
    int per_cu = 0, cus = 0;
    const size_t lds = (size_t)XQ_ROWS * a.H + sizeof(float) * (size_t)XQ_ROWS * (a.H / 32);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_layer_fused<WB, TT, NPG, NPD>,
                                                     256, lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 1;
    workers[dev] = per_cu * cus;
  }
  const size_t lds = (size_t)a.xq_rows * a.H + sizeof(float) * (size_t)a.xq_rows * (a.H / 32);
  launch_k(k_layer_fused<WB, TT, NPG, NPD>, dim3(workers[dev]), dim3(256), (uint32_t)lds, st, ev,
           a);
}

template <int WB, int TT>
static void launch_lf_np(const LayerArgs &a, hipStream_t st, Ev ev) {
  const int per = 128 / WB;
  const int ng = (a.H / per + 63) / 64, nd = (a.I / per + 63) / 64;
  if (ng <= 1 && nd <= 1) launch_lf<WB, TT, 1, 1>(a, st, ev);
  else if (ng <= 2 && nd <= 1) launch_lf<WB, TT, 2, 1>(a, st, ev);
  else if (ng <= 3 && nd <= 1) launch_lf<WB, TT, 3, 1>(a, st, ev);
  else if (ng <= 4 && nd <= 1) launch_lf<WB, TT, 4, 1>(a, st, ev);
  else launch_lf<WB, TT, 4, 2>(a, st, ev);
}

void launch_layer_fused(LayerArgs a, hipStream_t st, const moe_events *ev) {
  a.n_router = (a.E + 1) / 2;
  a.xq_rows = a.T < XQ_ROWS ? a.T : XQ_ROWS;
  a.n_slots_ub = a.n_shared + (a.T * a.K < a.E ? a.T * a.K : a.E);
  a.nw_gu = a.nw_dn = 0;
  const Ev e = stage_ev(ev, MOE_STAGE_FUSED);
  if (a.wbits == 4) {
    if (a.T == 1) launch_lf_np<4, 1>(a, st, e);
    else launch_lf_np<4, 4>(a, st, e);
  } else {
    if (a.T == 1) launch_lf_np<2, 1>(a, st, e);
    else launch_lf_np<2, 4>(a, st, e);
  }
}

}  // namespace moe

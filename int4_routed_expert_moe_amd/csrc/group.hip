// Batch-union grouping of token slots by expert.
//
// "Show HN: 遅いコンピュータで GLM 5.2 を実行する" (section 実装済みの主な機能,
// batch-union MoE item) reads each distinct expert of a batch once and applies
// it to every position routed to it; "Comment exécuter un réseau de neurones
// de 744 milliards de paramètres…" (section "Comment fonctionne le moteur")
// merges requests for the same expert.  This kernel produces the per-expert
// slot lists that let the FFN kernels stream each expert's weights once.
//
// Stable counting sort in one workgroup of 16 waves (E <= 1024, one expert
// per thread for the scans).  Wave w owns a contiguous range of slots.
// Positions are computed, never raced for:
//   pos(s) = offsets[e] + (slots of e in earlier waves' ranges)
//          + (slots of e earlier in this wave's range)
// so each expert's list is in increasing slot order and the result is
// bit-identical from run to run.  LDS atomics only count.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int GW = 16;  // waves per group workgroup
constexpr int PB = 8;   // slots per lane loaded together

// Exclusive prefix sum over the 1024 threads of the block; *total receives
// the sum of all v.  Every thread must call it (contains barriers).
__device__ int block_exscan(int v, int *wtot, int *total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wtot[wv] = x;
  __syncthreads();
  int pre = 0, all = 0;
  for (int w = 0; w < GW; w++) {
    const int t = wtot[w];
    pre += (w < wv) ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return pre + x - v;
}

__global__ void __launch_bounds__(GW * 64) k_group(int n_slots, int E,
                                                   const int32_t *__restrict__ idx,
                                                   int32_t *__restrict__ counts,
                                                   int32_t *__restrict__ offsets,
                                                   int32_t *__restrict__ perm,
                                                   int32_t *__restrict__ inv,
                                                   int32_t *__restrict__ active,
                                                   int32_t *__restrict__ n_active) {
  extern __shared__ int32_t lds[];
  int32_t *hist = lds;          // [GW][E]: per-wave counts, then per-wave cursors
  int32_t *off = lds + GW * E;  // [E] offsets
  __shared__ int32_t wtot[GW];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n_slots + GW - 1) / GW;
  const int s_lo = min(n_slots, wv * per);
  const int s_hi = min(n_slots, s_lo + per);

  for (int i = tid; i < GW * E; i += GW * 64) hist[i] = 0;
  __syncthreads();
  // idx in batches of PB slots per lane, each batch's loads in one round trip
  for (int base = s_lo; base < s_hi; base += 64 * PB) {
    int ev[PB];
#pragma unroll
    for (int u = 0; u < PB; u++) {
      const int s = base + 64 * u + lane;
      ev[u] = s < s_hi ? idx[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < PB; u++)
      if (ev[u] >= 0 && ev[u] < E) atomicAdd(&hist[wv * E + ev[u]], 1);
  }
  __syncthreads();
  int c = 0;
  if (tid < E) {
    for (int w = 0; w < GW; w++) {
      const int h = hist[w * E + tid];
      hist[w * E + tid] = c;  // slots of this expert in earlier waves' ranges
      c += h;
    }
  }
  int n_used = 0, n_act = 0;
  const int ex_c = block_exscan(c, wtot, &n_used);
  const int ex_a = block_exscan(c > 0 ? 1 : 0, wtot, &n_act);
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = ex_c;
    off[tid] = ex_c;
    active[tid] = -1;
  }
  if (tid == 0) {
    offsets[E] = n_used;
    n_active[0] = n_act;
  }
  for (int i = n_used + tid; i < n_slots; i += GW * 64) perm[i] = -1;  // unrouted tail
  __syncthreads();  // active[] = -1 is ordered before the compaction below
  if (tid < E && c > 0) active[ex_a] = tid;

  // Stable placement, 64 slots at a time in slot order.  Only wave wv touches
  // its cursors hist[wv][*], and a wave's LDS accesses are performed in
  // program order, so no barrier is needed inside this (wave-divergent) loop.
  for (int base = s_lo; base < s_hi; base += 64 * PB) {
    int ev[PB];
#pragma unroll
    for (int u = 0; u < PB; u++) {
      const int s = base + 64 * u + lane;
      ev[u] = s < s_hi ? idx[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < PB; u++) {
      const int s = base + 64 * u + lane;
      const int e = (ev[u] >= 0 && ev[u] < E) ? ev[u] : -1;
      // lanes holding the same expert: the valid lanes that agree with e on
      // each of its 10 bits (E <= 1024)
      unsigned long long m = __ballot(e >= 0);
#pragma unroll
      for (int b = 0; b < 10; b++) {
        const bool bit = (e >> b) & 1;
        const unsigned long long bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      const int rank = __popcll(m & ((1ull << lane) - 1ull));  // same expert, earlier lanes
      const int same = __popcll(m);
      int pos = 0;
      if (e >= 0) pos = off[e] + hist[wv * E + e] + rank;
      __builtin_amdgcn_wave_barrier();
      if (e >= 0) {
        perm[pos] = s;
        inv[s] = pos;
        if (rank == 0) hist[wv * E + e] += same;  // the first lane holding e advances
      } else if (s < s_hi) {
        inv[s] = -1;  // not routed (top-p drop)
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

void launch_group(int n_slots, int E, const int32_t *idx, int32_t *counts, int32_t *offsets,
                  int32_t *perm, int32_t *inv, int32_t *active, int32_t *n_active,
                  hipStream_t st, const moe_events *ev) {
  const size_t lds = sizeof(int32_t) * ((size_t)GW * E + E);
  launch_k(k_group, dim3(1), dim3(GW * 64), (uint32_t)lds, st, stage_ev(ev, MOE_STAGE_GROUP),
           n_slots, E, idx, counts, offsets, perm, inv, active, n_active);
}

}  // namespace moe

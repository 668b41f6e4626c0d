// The small-batch layer step (1..16 tokens) as moe_layer runs it in
// production; the kernels themselves are in decode.h.
#include "decode.h"

namespace moe {

size_t small_batch_slot_ints(int T, int K, int n_shared) {
  return (size_t)(n_shared + T * K) * SLOT_W;
}

// largest FP8 batch on the small-batch kernels: they take one token per
// chunk, so every token converts the codes again and larger batches turn
// VALU-bound (measured at 4 tokens: 251 against 254 us per step on the vector
// kernels; at 16: 886 against 791 us), where the vector kernels win
#ifndef MOE_F8_SMALL_T_MAX
#define MOE_F8_SMALL_T_MAX 4
#endif

bool small_batch_supported(const moe_cfg &c, int T) {
  if (T < 1 || T > MOE_SMALL_T_MAX) return false;
  // FP8: its 128x128 block scales of one 128-row block staged per gate/up
  // workgroup (at most 64 of them per matrix)
  if (c.wfmt == 2 && (c.hidden % 128 || c.inter % 128 || c.hidden / 128 > 64)) return false;
  if (c.wfmt == 2 && T > MOE_F8_SMALL_T_MAX) return false;
  if (T * c.top_k > 256) return false;
  if (c.hidden / 64 > 128 || c.hidden % sbk::RT) return false;
  const int per = 128 / c.wbits;  // codes per 16-byte piece
  return c.hidden / per <= (c.wbits == 8 ? 448 : 256) && c.inter / per <= 128;
}

void launch_small_batch(LayerArgs a, hipStream_t st, const moe_events *ev) {
  launch_small_batch_t<false>(a, st, ev);
}

// Group-limited top-k of token blockIdx.x by the whole workgroup (ranks in
// LDS), the selection the small-batch path runs: the chained path's
// selection at every batch size.
__global__ void __launch_bounds__(256) k_select_tokens(LayerArgs a) {
  __shared__ SelLds sm;
  select_token(a, sm, blockIdx.x);
}

void launch_router_select(const moe_cfg &c, int T, const float *s, const float *sb,
                          int32_t *idx, float *w, hipStream_t st, const moe_events *ev) {
  LayerArgs a{};
  a.E = c.n_experts;
  a.G = c.n_group;
  a.TG = c.topk_group;
  a.K = c.top_k;
  a.T = T;
  a.scale = c.routed_scaling;
  a.top_p = c.top_p;
  a.s = const_cast<float *>(s);  // read only
  a.sb = const_cast<float *>(sb);
  a.idx = idx;
  a.w = w;
  launch_k(k_select_tokens, dim3(T), dim3(256), 0, st, stage_ev(ev, MOE_STAGE_ROUTER_SELECT), a);
}

}  // namespace moe

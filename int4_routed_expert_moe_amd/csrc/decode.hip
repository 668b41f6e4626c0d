// The small-batch layer step (1..16 tokens) as moe_layer runs it in
// production; the kernels themselves are in decode.h.
#include "decode.h"

namespace moe {

size_t small_batch_slot_ints(int T, int K, int n_shared) {
  return (size_t)(n_shared + T * K) * SLOT_W;
}

bool small_batch_supported(const moe_cfg &c, int T) {
  if (T < 1 || T > MOE_SMALL_T_MAX) return false;
  if (c.wfmt == 2) return false;  // FP8 experts take the chained path
  if (T * c.top_k > 256) return false;
  if (c.hidden / 64 > 128 || c.hidden % sbk::RT) return false;
  const int per = 128 / c.wbits;  // codes per 16-byte piece
  return c.hidden / per <= (c.wbits == 8 ? 448 : 256) && c.inter / per <= 128;
}

void launch_small_batch(LayerArgs a, hipStream_t st, const moe_events *ev) {
  launch_small_batch_t<false>(a, st, ev);
}

}  // namespace moe

// The small-batch layer step with its intermediates written to a
// moe_layer_debug (Q8_0 of x, the batch union, the exact int32 block dots of
// gate/up and down, h, Q8_0 of h): the same kernels as decode.hip (decode.h)
// compiled with their dump stores on.
#include "decode.h"

namespace moe {

void launch_small_batch_dbg(LayerArgs a, hipStream_t st, const moe_events *ev) {
  launch_small_batch_t<true>(a, st, ev);
}

}  // namespace moe

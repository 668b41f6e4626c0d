// Work items of the grouped expert GEMMs (ffn_mfma.hip, ffn_rows.hip):
// (expert, first position in its token list, token count) from the tile list
// that k_mfma_tiles builds out of the grouping offsets, and the small helpers
// both files share.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int TILE_T = 64;  // tokens per work item

struct TileInfo {
  const uint8_t *blob;
  int n;         // tokens in the tile
  bool shared;
};

__device__ __forceinline__ TileInfo tile_info(const FfnArgs &a, int4 t) {
  TileInfo r;
  r.shared = t.x >= a.E;
  r.blob = r.shared ? a.shared : expert_record(a, min(max(t.x, 0), a.E - 1));
  r.n = min(max(t.z, 0), TILE_T);
  return r;
}

// token and pair of list position i of a tile
__device__ __forceinline__ void tile_tok(const FfnArgs &a, int4 t, bool shared, int i, int &tok,
                                         int &pair) {
  if (shared) {
    tok = min(max(t.y + i, 0), a.T - 1);
    pair = a.T * a.K + tok;
  } else {
    const int sl = min(max(a.perm[min(max(t.y + i, 0), a.T * a.K - 1)], 0), a.T * a.K - 1);
    tok = sl / a.K;
    pair = sl;
  }
}

// 8 activation bytes reordered (even positions, then odd) to match the
// nibble split of the weights.
__device__ __forceinline__ uint2 even_odd8(uint32_t w0, uint32_t w1) {
  return make_uint2((uint32_t)even_bytes(w0, w1), (uint32_t)odd_bytes(w0, w1));
}

}  // namespace moe

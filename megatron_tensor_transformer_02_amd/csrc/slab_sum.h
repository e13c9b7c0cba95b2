// Fixed-order sums of per-slab partial rows: out[c] = sum over s of
// partial[s * w + c] (the second stage of the deterministic column sums:
// bias gradients, LayerNorm dgamma / dbeta).
#pragma once
#include "common.h"

namespace mp {

// A block of SLAB_COLS x SLAB_GROUPS threads owns SLAB_COLS consecutive
// columns.  Group q sums slabs q, q + SLAB_GROUPS, ... in ascending order,
// eight loads in flight per thread; the group sums are then added in group
// order.  With few slabs per group the loads of a column are all in flight
// at once.  The order depends only on the slab count, so results are
// identical run to run.
constexpr int SLAB_COLS = 32, SLAB_GROUPS = 32, SLAB_THREADS = SLAB_COLS * SLAB_GROUPS;

// Returns the sum of column c in threads of group 0 (0 elsewhere); every
// thread of the block must call it (it holds one barrier).
__device__ __forceinline__ float slab_column_sum(const float* __restrict__ partial, int64_t slabs, int64_t w,
                                                 int64_t c, float (*red)[SLAB_COLS]) {
  const int cl = threadIdx.x % SLAB_COLS, q = threadIdx.x / SLAB_COLS;
  float t = 0.0f;
  if (c < w) {
    for (int64_t s0 = q; s0 < slabs; s0 += 8 * SLAB_GROUPS) {
      float a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t s = s0 + static_cast<int64_t>(i) * SLAB_GROUPS;
        a[i] = s < slabs ? partial[s * w + c] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) t += a[i];
    }
  }
  red[q][cl] = t;
  __syncthreads();
  float v = 0.0f;
  if (q == 0) {
    v = red[0][cl];
#pragma unroll
    for (int i = 1; i < SLAB_GROUPS; ++i) v += red[i][cl];
  }
  return v;
}

}  // namespace mp

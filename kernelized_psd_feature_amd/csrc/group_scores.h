// Scores of (query, key) pairs for the fp32 kernels, with a fast path for a single feature
// group: the group helpers of device.h handle any grouping through per-coordinate bit tests;
// with one group (the plain ψ(u) = u u^T) the score is one dot product, squared.  Both paths
// evaluate the same fused multiply-adds in the same order, so results are bitwise those of the
// group helpers.
#pragma once

#include "device.h"

namespace kata {

// grouped_square with the single-group case as one dot product
template <int P, typename Y>
__device__ __forceinline__ float score_square(const float (&x)[P], const Y& y, Groups g) {
  if (g.start == 1u) {                            // one group (uniform across the launch)
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) d = fmaf(x[i], y[i], d);
    return fmaf(d, d, 0.f);
  }
  return grouped_square(x, y, g);
}

// grouped_dots with the single-group case as one dot product: sc[i] = x . y for every i
template <int P, typename Y>
__device__ __forceinline__ float score_dots(const float (&x)[P], const Y& y, Groups g,
                                            float (&sc)[P]) {
  if (g.start == 1u) {
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) d = fmaf(x[i], y[i], d);
#pragma unroll
    for (int i = 0; i < P; ++i) sc[i] = d;
    return fmaf(d, d, 0.f);
  }
  return grouped_dots(x, y, g, sc);
}

}  // namespace kata

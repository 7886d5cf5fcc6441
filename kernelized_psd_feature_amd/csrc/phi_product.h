// fp32 chunk products with the rank-one PSD feature phi_f(x) = x_i x_j (f = i p + j), formed
// on the fly, shared by the fp32 chunk-state kernel of the forward and the reverse-state
// kernel of the chunked backward:
//
//   out[d][f]  = sum_{s < C} phi_f(x_s) y_s[d]     (d < dv)
//   out[dv][f] = sum_{s < C} phi_f(x_s) w_s        (w_s = 1 where kOnes)
//
// with phi_f = 0 for pairs across KATA-Mg groups (selection, so a non-finite x or y never
// reaches those rows).  Work item (fq, dq): the four features (i, 4 jq .. 4 jq + 3) of feature
// quad fq = i p / 4 + jq, times the columns [16 dq, 16 dq + 16); items with dq == 0 also carry
// the w column.  Per row s: 6 LDS reads (broadcasts within a wave) for 4 products and 68 FMAs.
// Each output sums over s in order, as a plain loop would.
#pragma once

#include "device.h"

namespace kata {

template <int P, int DV, bool kOnes>
__device__ __forceinline__ void phi_product(const float (*xs)[P], const float (*ys)[DV],
                                            const float* ws, int C, int gs, float* out) {
  constexpr int PP = P * P, NFQ = PP / 4, NDQ = DV / 16;
  static_assert(DV % 16 == 0 && P % 4 == 0, "phi product tiling");
  for (int item = threadIdx.x; item < NFQ * NDQ; item += blockDim.x) {
    const int fq = item % NFQ, dq = item / NFQ;
    const int i = fq / (P / 4), j0 = 4 * (fq % (P / 4)), f0 = i * P + j0;
    bool in[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) in[x] = same_group(i, j0 + x, gs);
    float acc[4][16], wacc[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      wacc[x] = 0.f;
#pragma unroll
      for (int y = 0; y < 16; ++y) acc[x][y] = 0.f;
    }
    for (int s = 0; s < C; ++s) {
      const float xi = xs[s][i];
      const float4 xj = *reinterpret_cast<const float4*>(&xs[s][j0]);
      const float xjs[4] = {xj.x, xj.y, xj.z, xj.w};
      float phi[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) phi[x] = in[x] ? xi * xjs[x] : 0.f;
      float yy[16];
#pragma unroll
      for (int y4 = 0; y4 < 4; ++y4) {
        const float4 u = *reinterpret_cast<const float4*>(&ys[s][16 * dq + 4 * y4]);
        yy[4 * y4] = u.x; yy[4 * y4 + 1] = u.y; yy[4 * y4 + 2] = u.z; yy[4 * y4 + 3] = u.w;
      }
      const float wsv = kOnes ? 1.f : ws[s];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        wacc[x] = fmaf(phi[x], wsv, wacc[x]);
#pragma unroll
        for (int y = 0; y < 16; ++y) acc[x][y] = fmaf(phi[x], yy[y], acc[x][y]);
      }
    }
    // rows across groups are exact zeros
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      wacc[x] = in[x] ? wacc[x] : 0.f;
#pragma unroll
      for (int y = 0; y < 16; ++y) acc[x][y] = in[x] ? acc[x][y] : 0.f;
    }
#pragma unroll
    for (int y = 0; y < 16; ++y)
      *reinterpret_cast<float4*>(out + (long long)(16 * dq + y) * PP + f0) =
          float4{acc[0][y], acc[1][y], acc[2][y], acc[3][y]};
    if (dq == 0)
      *reinterpret_cast<float4*>(out + (long long)DV * PP + f0) =
          float4{wacc[0], wacc[1], wacc[2], wacc[3]};
  }
}

// Features [f0, f0 + FB) of a state stored [dv + 1][p^2] (d-major), staged into LDS as
// [feature][SROW] rows, column dv holding the last state row (Z or r), through registers:
// load() issues the global reads (coalesced over features) and store() writes LDS, so the
// next block's reads can be in flight while the current block is computed.  NT threads.
template <int PP, int DV, int FB, int SROW, int NT>
struct StateBlock {
  static constexpr int kVals = (DV + 1) * FB, N = (kVals + NT - 1) / NT;
  float r[N];
  __device__ __forceinline__ void load(const float* __restrict__ S, int f0) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int e = threadIdx.x + n * NT;
      if (e < kVals) r[n] = S[(long long)(e / FB) * PP + f0 + e % FB];
    }
  }
  __device__ __forceinline__ void store(float (*sl)[SROW]) const {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int e = threadIdx.x + n * NT;
      if (e < kVals) sl[e % FB][e / FB] = r[n];
    }
  }
};

}  // namespace kata

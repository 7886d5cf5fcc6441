// fp32 backward of the causal normalized attention with squared scores, for gfx950.
//
// Forward (gist.science sections 2.1-2.2): s_ts = q_t . k_s, a_ts = s_ts^2 (s <= t),
// D_t = eps + sum_s a_ts, o_t = sum_s a_ts v_s / D_t.  For L = sum_t <dO_t, o_t>
// (derived here; the KATA README names a flash backward, the pages print no formula):
//   delta_t = dO_t . o_t,   G_ts = (dO_t . v_s - delta_t) / D_t
//   dq_t = sum_{s<=t} 2 s_ts G_ts k_s,   dk_s = sum_{t>=s} 2 s_ts G_ts q_t,
//   dv_s = sum_{t>=s} a_ts dO_t / D_t.
// Every quantity is fp32: D_t can be as small as eps, where G grows like 1/D_t, so no
// intermediate is rounded to bf16.
//
// Three kernels: prep (D_t and delta_t per row, a flash-style forward), dq (one thread per
// query, keys streamed through LDS) and dk/dv (one thread per key, queries streamed).
#include "device.h"
#include "group_scores.h"

namespace kata {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;

// D and delta are fp32 [B][H][T].
__device__ __forceinline__ long long bht(const DevProblem& pr, int b, int h, int t) {
  return ((long long)b * pr.H + h) * pr.T + t;
}

template <typename Tin, int P, int DV>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(
    DevProblem pr, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ dO, float* __restrict__ Dout,
    float* __restrict__ delta) {
  constexpr int DP = DV / 4;
  __shared__ float ks[kRows][P];
  __shared__ float vs[kRows][DV];
  __shared__ float red[4][kRows];
  const int b = blockIdx.z, h = blockIdx.y, t0 = blockIdx.x * kRows;
  const int row = threadIdx.x % kRows, part = threadIdx.x / kRows;
  const int t = t0 + row;
  float qr[P];
#pragma unroll
  for (int i = 0; i < P; ++i) qr[i] = t < pr.T ? to_f32(q[row_off(pr.sq, b, t, h) + i]) : 0.f;
  float acc[DP];
#pragma unroll
  for (int j = 0; j < DP; ++j) acc[j] = 0.f;
  float l = 0.f;
  const Groups grp = make_groups(P, pr.gs);
  const int kend = min(pr.T, t0 + kRows);
  for (int s0 = 0; s0 < kend; s0 += kRows) {
    __syncthreads();
    for (int e = threadIdx.x; e < kRows * P; e += kThreads) {
      int s = e / P, i = e % P, ss = s0 + s;
      ks[s][i] = ss < pr.T ? to_f32(k[row_off(pr.sk, b, ss, h) + i]) : 0.f;
    }
    for (int e = threadIdx.x; e < kRows * DV; e += kThreads) {
      int s = e / DV, d = e % DV, ss = s0 + s;
      vs[s][d] = ss < pr.T ? to_f32(v[row_off(pr.sv, b, ss, h) + d]) : 0.f;
    }
    __syncthreads();
    const int smax = min(kRows, kend - s0);
    for (int s = 0; s < smax; ++s) {
      if (s0 + s <= t) {
        const float a = score_square(qr, ks[s], grp);
        l += a;
#pragma unroll
        for (int j = 0; j < DP; ++j) acc[j] = fmaf(a, vs[s][part * DP + j], acc[j]);
      }
    }
  }
  const float D = pr.eps + l;
  float part_delta = 0.f;
  if (t < pr.T) {
    const Tin* gp = dO + row_off(pr.sdo, b, t, h) + part * DP;
#pragma unroll
    for (int j = 0; j < DP; ++j) part_delta = fmaf(to_f32(gp[j]), acc[j] / D, part_delta);
  }
  red[part][row] = part_delta;
  __syncthreads();
  if (part == 0 && t < pr.T) {
    Dout[bht(pr, b, h, t)] = D;
    delta[bht(pr, b, h, t)] = ((red[0][row] + red[1][row]) + red[2][row]) + red[3][row];
  }
}

// dq: one thread per query row; keys streamed through LDS in tiles of 64.
template <typename Tin, int P, int DV>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(
    DevProblem pr, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ dO, const float* __restrict__ Din,
    const float* __restrict__ delta, float* __restrict__ dq) {
  __shared__ float ks[kRows][P];
  __shared__ float vs[kRows][DV];
  const int b = blockIdx.z, h = blockIdx.y, t0 = blockIdx.x * kThreads;
  const int t = t0 + threadIdx.x;
  const bool live = t < pr.T;
  float qr[P], g[DV], acc[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    qr[i] = live ? to_f32(q[row_off(pr.sq, b, t, h) + i]) : 0.f;
    acc[i] = 0.f;
  }
#pragma unroll
  for (int d = 0; d < DV; ++d) g[d] = live ? to_f32(dO[row_off(pr.sdo, b, t, h) + d]) : 0.f;
  const float invD = live ? 1.f / Din[bht(pr, b, h, t)] : 0.f;
  const float dl = live ? delta[bht(pr, b, h, t)] : 0.f;
  const Groups grp = make_groups(P, pr.gs);
  const int kend = min(pr.T, t0 + kThreads);
  for (int s0 = 0; s0 < kend; s0 += kRows) {
    __syncthreads();
    for (int e = threadIdx.x; e < kRows * P; e += kThreads) {
      int s = e / P, i = e % P, ss = s0 + s;
      ks[s][i] = ss < pr.T ? to_f32(k[row_off(pr.sk, b, ss, h) + i]) : 0.f;
    }
    for (int e = threadIdx.x; e < kRows * DV; e += kThreads) {
      int s = e / DV, d = e % DV, ss = s0 + s;
      vs[s][d] = ss < pr.T ? to_f32(v[row_off(pr.sv, b, ss, h) + d]) : 0.f;
    }
    __syncthreads();
    const int smax = min(kRows, kend - s0);
    for (int s = 0; s < smax; ++s) {
      if (live && s0 + s <= t) {
        float sc[P], gv = 0.f;
        score_dots(qr, ks[s], grp, sc);
#pragma unroll
        for (int d = 0; d < DV; ++d) gv = fmaf(g[d], vs[s][d], gv);
        const float G = (gv - dl) * invD;
#pragma unroll
        for (int i = 0; i < P; ++i) acc[i] = fmaf(2.f * sc[i] * G, ks[s][i], acc[i]);
      }
    }
  }
  if (live) {
    float* op = dq + row_off(pr.sq, b, t, h);
#pragma unroll
    for (int i = 0; i < P; ++i) op[i] = acc[i];
  }
}

// dk, dv: one thread per key row; queries t >= s streamed through LDS in tiles of 64.
template <typename Tin, int P, int DV>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(
    DevProblem pr, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ dO, const float* __restrict__ Din,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv) {
  __shared__ float qs[kRows][P];
  __shared__ float gs[kRows][DV];
  __shared__ float invD[kRows];
  __shared__ float dls[kRows];
  const int b = blockIdx.z, h = blockIdx.y, s_base = blockIdx.x * kThreads;
  const int s = s_base + threadIdx.x;
  const bool live = s < pr.T;
  float kr[P], vr[DV], ak[P], av[DV];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    kr[i] = live ? to_f32(k[row_off(pr.sk, b, s, h) + i]) : 0.f;
    ak[i] = 0.f;
  }
#pragma unroll
  for (int d = 0; d < DV; ++d) {
    vr[d] = live ? to_f32(v[row_off(pr.sv, b, s, h) + d]) : 0.f;
    av[d] = 0.f;
  }
  const Groups grp = make_groups(P, pr.gs);
  for (int q0 = s_base; q0 < pr.T; q0 += kRows) {     // queries t >= s_base
    __syncthreads();
    for (int e = threadIdx.x; e < kRows * P; e += kThreads) {
      int r = e / P, i = e % P, tt = q0 + r;
      qs[r][i] = tt < pr.T ? to_f32(q[row_off(pr.sq, b, tt, h) + i]) : 0.f;
    }
    for (int e = threadIdx.x; e < kRows * DV; e += kThreads) {
      int r = e / DV, d = e % DV, tt = q0 + r;
      gs[r][d] = tt < pr.T ? to_f32(dO[row_off(pr.sdo, b, tt, h) + d]) : 0.f;
    }
    if (threadIdx.x < kRows) {
      int tt = q0 + threadIdx.x;
      invD[threadIdx.x] = tt < pr.T ? 1.f / Din[bht(pr, b, h, tt)] : 0.f;
      dls[threadIdx.x] = tt < pr.T ? delta[bht(pr, b, h, tt)] : 0.f;
    }
    __syncthreads();
    const int rmax = min(kRows, pr.T - q0);
    for (int r = 0; r < rmax; ++r) {
      if (live && q0 + r >= s) {
        float sc[P], gv = 0.f;
        const float a = score_dots(kr, qs[r], grp, sc);
#pragma unroll
        for (int d = 0; d < DV; ++d) gv = fmaf(gs[r][d], vr[d], gv);
        const float G = (gv - dls[r]) * invD[r];
        const float w = a * invD[r];
#pragma unroll
        for (int i = 0; i < P; ++i) ak[i] = fmaf(2.f * sc[i] * G, qs[r][i], ak[i]);
#pragma unroll
        for (int d = 0; d < DV; ++d) av[d] = fmaf(w, gs[r][d], av[d]);
      }
    }
  }
  if (live) {
    float* kp = dk + row_off(pr.sk, b, s, h);
    float* vp = dv + row_off(pr.sv, b, s, h);
#pragma unroll
    for (int i = 0; i < P; ++i) kp[i] = ak[i];
#pragma unroll
    for (int d = 0; d < DV; ++d) vp[d] = av[d];
  }
}

template <template <typename, int, int> class Launch, typename... Args>
hipError_t dispatch_in(int p, int dv, bool in_bf16, Args&&... args) {
#define KATA_CASE(P_, DV_)                                                       \
  if (p == P_ && dv == DV_) {                                                    \
    if (in_bf16) return Launch<__bf16, P_, DV_>::run(args...);                   \
    return Launch<float, P_, DV_>::run(args...);                                 \
  }
  KATA_CASE(8, 16) KATA_CASE(8, 64) KATA_CASE(16, 16) KATA_CASE(16, 64) KATA_CASE(32, 16)
  KATA_CASE(32, 64)
#undef KATA_CASE
  return hipErrorInvalidValue;
}

template <typename Tin, int P, int DV>
struct PrepLaunch {
  static hipError_t run(const DevProblem& pr, const void* q, const void* k, const void* v,
                        const void* dO, float* D, float* delta, hipStream_t st) {
    dim3 grid((pr.T + kRows - 1) / kRows, pr.H, pr.B);
    launch_kernel(bwd_prep_kernel<Tin, P, DV>, grid, kThreads, 0, st,
        pr, (const Tin*)q, (const Tin*)k, (const Tin*)v, (const Tin*)dO, D, delta);
    return hipGetLastError();
  }
};

template <typename Tin, int P, int DV>
struct DqLaunch {
  static hipError_t run(const DevProblem& pr, const void* q, const void* k, const void* v,
                        const void* dO, const float* D, const float* delta, float* dq,
                        hipStream_t st) {
    dim3 grid((pr.T + kThreads - 1) / kThreads, pr.H, pr.B);
    launch_kernel(bwd_dq_kernel<Tin, P, DV>, grid, kThreads, 0, st,
        pr, (const Tin*)q, (const Tin*)k, (const Tin*)v, (const Tin*)dO, D, delta, dq);
    return hipGetLastError();
  }
};

template <typename Tin, int P, int DV>
struct DkdvLaunch {
  static hipError_t run(const DevProblem& pr, const void* q, const void* k, const void* v,
                        const void* dO, const float* D, const float* delta, float* dk,
                        float* dv, hipStream_t st) {
    dim3 grid((pr.T + kThreads - 1) / kThreads, pr.H, pr.B);
    launch_kernel(bwd_dkdv_kernel<Tin, P, DV>, grid, kThreads, 0, st,
        pr, (const Tin*)q, (const Tin*)k, (const Tin*)v, (const Tin*)dO, D, delta, dk, dv);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_bwd_prep(const DevProblem& pr, bool in_bf16, const void* q, const void* k,
                           const void* v, const void* dO, float* D, float* delta,
                           hipStream_t st) {
  return dispatch_in<PrepLaunch>(pr.p, pr.dv, in_bf16, pr, q, k, v, dO, D, delta, st);
}

hipError_t launch_bwd_dq(const DevProblem& pr, bool in_bf16, const void* q, const void* k,
                         const void* v, const void* dO, const float* D, const float* delta,
                         float* dq, hipStream_t st) {
  return dispatch_in<DqLaunch>(pr.p, pr.dv, in_bf16, pr, q, k, v, dO, D, delta, dq, st);
}

hipError_t launch_bwd_dkdv(const DevProblem& pr, bool in_bf16, const void* q, const void* k,
                           const void* v, const void* dO, const float* D, const float* delta,
                           float* dk, float* dv, hipStream_t st) {
  return dispatch_in<DkdvLaunch>(pr.p, pr.dv, in_bf16, pr, q, k, v, dO, D, delta, dk, dv,
                                 st);
}

}  // namespace kata

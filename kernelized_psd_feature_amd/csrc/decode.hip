// Recurrent form of the attention for gfx950: the state (S, Z) is carried token by token.
//
//   S_t = S_{t-1} + phi(k_t) v_t^T,  Z_t = Z_{t-1} + k_t k_t^T,
//   o_t = phi(q_t)^T S_t / (eps + q_t^T Z_t q_t),   phi(u) = vec(u u^T)
//
// (gist.science "Technische Samenvatting", section 2.2 for psi(u) = u u^T and section 2.1 for
// the normalized readout; ai.info "AI summary", Main Findings, the bullet on constant-state
// recurrent inference.)  The state of one (b, h) is the fp32 array [dv + 1][p^2]: row d < dv
// holds S[(i, j)][d] at column i p + j, row dv holds Z[i][j] at column i p + j.
//
// Decode is bound by the state traffic (one read and one write of (dv + 1) p^2 floats per
// (b, h) and call), so the kernels spread every state row over one wave's 64 lanes: lane l
// holds the E = p^2 / 64 consecutive features E l .. E l + E - 1 of its row, which share the
// factor index i = E l / p (E divides p) and have consecutive j.  Reads and writes of a row
// are then single coalesced 1 KB (p = 16) transactions.
#include "device.h"

namespace kata {
namespace {

constexpr int kWaves = 4;                 // state rows per workgroup
constexpr int kThreads = 64 * kWaves;

template <int N>
__device__ __forceinline__ void load_run(float (&x)[N], const float* p) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int r = 0; r < N; r += 4) {
      const float4 u = *reinterpret_cast<const float4*>(p + r);
      x[r] = u.x; x[r + 1] = u.y; x[r + 2] = u.z; x[r + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int r = 0; r < N; ++r) x[r] = p[r];
  }
}

template <int N>
__device__ __forceinline__ void store_run(float* p, const float (&x)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int r = 0; r < N; r += 4)
      *reinterpret_cast<float4*>(p + r) = float4{x[r], x[r + 1], x[r + 2], x[r + 3]};
  } else {
#pragma unroll
    for (int r = 0; r < N; ++r) p[r] = x[r];
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// Rows d < dv of the state, one wave per row.  Grid (dv / 4, H, B).  Every wave also carries
// its own register copy of the Z row (read, never written here) for the denominator; the Z
// row itself is advanced by decode_z_kernel, which runs after this kernel on the stream.
template <typename Tin, typename Tout, int P, int DV>
__global__ __launch_bounds__(kThreads) void decode_rows_kernel(
    DevProblem pr, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den,
    float* __restrict__ state) {
  constexpr int PP = P * P, E = PP / 64;
  const int lane = threadIdx.x & 63, d = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int h = blockIdx.y, b = blockIdx.z;
  const int f0 = E * lane, i = f0 / P, j0 = f0 % P;
  float* st = state + ((long long)b * pr.H + h) * (long long)(DV + 1) * PP;
  float s[E], z[E];
  load_run(s, st + (long long)d * PP + f0);
  load_run(z, st + (long long)DV * PP + f0);
  unsigned in = 0;                                 // bit r: feature (i, j0 + r) is in a group
#pragma unroll
  for (int r = 0; r < E; ++r) in |= same_group(i, j0 + r, pr.gs) ? 1u << r : 0u;
  for (int t = 0; t < pr.T; ++t) {
    const Tin* qt = q + row_off(pr.sq, b, t, h);
    const Tin* kt = k + row_off(pr.sk, b, t, h);
    const float qi = to_f32(qt[i]), ki = to_f32(kt[i]);
    const float vd = to_f32(v[row_off(pr.sv, b, t, h) + d]);
    float kj[E], qj[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
      kj[r] = to_f32(kt[j0 + r]);
      qj[r] = to_f32(qt[j0 + r]);
    }
    float num = 0.f, zq = 0.f;
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const bool on = (in >> r) & 1u;
      const float kk = on ? ki * kj[r] : 0.f;        // phi_f(k_t)
      const float qq = on ? qi * qj[r] : 0.f;        // phi_f(q_t)
      s[r] = fmaf(kk, vd, s[r]);
      z[r] += kk;
      num = fmaf(qq, s[r], num);
      zq = fmaf(qq, z[r], zq);
    }
    num = wave_sum(num);
    zq = wave_sum(zq);
    const float D = pr.eps + zq;
    if (lane == 0) {
      o[row_off(pr.so, b, t, h) + d] = from_f32<Tout>(num / D);
      if (den && d == 0) den[((long long)b * pr.T + t) * pr.H + h] = D;
    }
  }
  store_run(st + (long long)d * PP + f0, s);
}

// Row dv (Z) of the state.  Grid (1, H, B), one wave.
template <typename Tin, int P, int DV>
__global__ __launch_bounds__(64) void decode_z_kernel(DevProblem pr, const Tin* __restrict__ k,
                                                      float* __restrict__ state) {
  constexpr int PP = P * P, E = PP / 64;
  const int lane = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int f0 = E * lane, i = f0 / P, j0 = f0 % P;
  float* zr = state + ((long long)b * pr.H + h) * (long long)(DV + 1) * PP + (long long)DV * PP + f0;
  float z[E];
  load_run(z, zr);
  unsigned in = 0;
#pragma unroll
  for (int r = 0; r < E; ++r) in |= same_group(i, j0 + r, pr.gs) ? 1u << r : 0u;
  for (int t = 0; t < pr.T; ++t) {
    const Tin* kt = k + row_off(pr.sk, b, t, h);
    const float ki = to_f32(kt[i]);
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const float kk = ki * to_f32(kt[j0 + r]);
      z[r] += ((in >> r) & 1u) ? kk : 0.f;
    }
  }
  store_run(zr, z);
}

// Fused form for p <= 16: one workgroup of 16 waves per (b, h) holds the whole state, so the
// Z row needs no second kernel.  Wave w owns the value rows d = w + 16 r (r < dv / 16) and
// keeps its own register copy of the Z row for the denominators; every wave has used that
// copy (so read the old Z) before the barrier, after which wave 0 alone writes the advanced
// Z row.  Grid (H, B), 1024 threads.
constexpr int kFusedWaves = 16;

template <typename Tin, typename Tout, int P, int DV>
__global__ __launch_bounds__(64 * kFusedWaves) void decode_fused_kernel(
    DevProblem pr, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den,
    float* __restrict__ state) {
  constexpr int PP = P * P, E = PP / 64, R = DV / kFusedWaves;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  const int f0 = E * lane, i = f0 / P, j0 = f0 % P;
  float* st = state + ((long long)b * pr.H + h) * (long long)(DV + 1) * PP;
  float s[R][E], z[E];
#pragma unroll
  for (int r = 0; r < R; ++r) load_run(s[r], st + (long long)(w + kFusedWaves * r) * PP + f0);
  load_run(z, st + (long long)DV * PP + f0);
  unsigned in = 0;                                 // bit e: feature (i, j0 + e) is in a group
#pragma unroll
  for (int e = 0; e < E; ++e) in |= same_group(i, j0 + e, pr.gs) ? 1u << e : 0u;
  for (int t = 0; t < pr.T; ++t) {
    const Tin* qt = q + row_off(pr.sq, b, t, h);
    const Tin* kt = k + row_off(pr.sk, b, t, h);
    const Tin* vt = v + row_off(pr.sv, b, t, h);
    const float qi = to_f32(qt[i]), ki = to_f32(kt[i]);
    float kk[E], qq[E], vd[R];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool on = (in >> e) & 1u;
      kk[e] = on ? ki * to_f32(kt[j0 + e]) : 0.f;    // phi_f(k_t)
      qq[e] = on ? qi * to_f32(qt[j0 + e]) : 0.f;    // phi_f(q_t)
    }
#pragma unroll
    for (int r = 0; r < R; ++r) vd[r] = to_f32(vt[w + kFusedWaves * r]);
    float zq = 0.f, num[R];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      z[e] += kk[e];
      zq = fmaf(qq[e], z[e], zq);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      num[r] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        s[r][e] = fmaf(kk[e], vd[r], s[r][e]);
        num[r] = fmaf(qq[e], s[r][e], num[r]);
      }
    }
    const float D = pr.eps + wave_sum(zq);
#pragma unroll
    for (int r = 0; r < R; ++r) num[r] = wave_sum(num[r]);
    if (lane == 0) {
      Tout* ot = o + row_off(pr.so, b, t, h);
#pragma unroll
      for (int r = 0; r < R; ++r) ot[w + kFusedWaves * r] = from_f32<Tout>(num[r] / D);
      if (den && w == 0) den[((long long)b * pr.T + t) * pr.H + h] = D;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) store_run(st + (long long)(w + kFusedWaves * r) * PP + f0, s[r]);
  __syncthreads();                                 // every wave has used its copy of the old Z
  if (w == 0) store_run(st + (long long)DV * PP + f0, z);
}

// Sum of n states per sequence, in order, into the [dv + 1][p^2] layout.  Grid
// (ceil(E / 4 / 256), n_seq); thread x sums float4 x of every state.  tiles != 0: the sources
// are the MFMA state kernel's accumulator layout for p = 16, dv = 64 (float4 x = tile t, value
// tile nt, lane l holds S[16 t + 4 (l / 16) + r][16 nt + l % 16], r = 0..3, and the Z tile
// after the 16 S tiles holds Z[4 (l / 16) + r][l % 16]), which is moved to its place here.
__global__ __launch_bounds__(256) void state_sum_kernel(const float* __restrict__ src,
                                                        long long n, long long elems,
                                                        int tiles, float* __restrict__ dst) {
  const long long x = (long long)blockIdx.x * 256 + threadIdx.x;
  if (4 * x >= elems) return;
  const long long seq = blockIdx.y;
  const float* p = src + seq * n * elems + 4 * x;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (long long c = 0; c < n; ++c) {
    const float4 u = *reinterpret_cast<const float4*>(p + c * elems);
    acc.x += u.x; acc.y += u.y; acc.z += u.z; acc.w += u.w;
  }
  long long off = 4 * x;
  if (tiles) {
    const int lane = int(x & 63), nt = int((x >> 6) & 3), t = int(x >> 8);   // t = 16 is Z
    const int g = lane >> 4, l16 = lane & 15;
    // S: row d = 16 nt + l16, features 16 t + 4 g ..;  Z (symmetric): row 64, features
    // 16 l16 + 4 g ..
    off = t < 16 ? (long long)(16 * nt + l16) * 256 + 16 * t + 4 * g : 64LL * 256 + 16 * l16 + 4 * g;
  }
  *reinterpret_cast<float4*>(dst + seq * elems + off) = acc;
}

template <typename Tin, typename Tout, int P, int DV>
hipError_t launch_decode_t(const DevProblem& pr, const void* q, const void* k, const void* v,
                           void* o, float* den, float* state, hipStream_t st) {
  static_assert(DV % kWaves == 0 && (P * P) % 64 == 0, "decode tiling");
  if constexpr (P <= 16 && DV % kFusedWaves == 0) {
    launch_kernel(decode_fused_kernel<Tin, Tout, P, DV>, dim3(pr.H, pr.B), 64 * kFusedWaves, 0,
                  st, pr, (const Tin*)q, (const Tin*)k, (const Tin*)v, (Tout*)o, den, state);
    return hipGetLastError();
  }
  launch_kernel(decode_rows_kernel<Tin, Tout, P, DV>, dim3(DV / kWaves, pr.H, pr.B), kThreads,
                0, st, pr, (const Tin*)q, (const Tin*)k, (const Tin*)v, (Tout*)o, den, state);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_kernel(decode_z_kernel<Tin, P, DV>, dim3(1, pr.H, pr.B), 64, 0, st, pr, (const Tin*)k,
                state);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DevProblem& pr, bool in_bf16, bool out_bf16, const void* q,
                         const void* k, const void* v, void* o, float* den, float* state,
                         hipStream_t st) {
#define KATA_CASE(P_, DV_)                                                                       \
  if (pr.p == P_ && pr.dv == DV_) {                                                              \
    if (in_bf16 && out_bf16) return launch_decode_t<__bf16, __bf16, P_, DV_>(pr, q, k, v, o, den, state, st); \
    if (in_bf16) return launch_decode_t<__bf16, float, P_, DV_>(pr, q, k, v, o, den, state, st); \
    return launch_decode_t<float, float, P_, DV_>(pr, q, k, v, o, den, state, st);               \
  }
  KATA_CASE(8, 16) KATA_CASE(8, 64) KATA_CASE(16, 16) KATA_CASE(16, 64) KATA_CASE(32, 16)
  KATA_CASE(32, 64)
#undef KATA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_state_sum(const float* src, long long n_seq, long long n, long long elems,
                            bool tiles, float* dst, hipStream_t st) {
  if (elems % 4 || (tiles && elems != 16 * 16 * 65)) return hipErrorInvalidValue;   // p^2 (dv + 1)
  const long long blocks = (elems / 4 + 255) / 256;
  launch_kernel(state_sum_kernel, dim3((unsigned)blocks, (unsigned)n_seq), 256, 0, st, src, n,
                elems, tiles ? 1 : 0, dst);
  return hipGetLastError();
}

}  // namespace kata

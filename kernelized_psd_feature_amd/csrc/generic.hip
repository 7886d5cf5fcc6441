// fp32-arithmetic VALU kernels for gfx950: the quadratic forward, the chunk-state build and
// chunk readout of the chunked forward (one segment per chunk), for every supported
// (p, dv, dtype).  They are the exact-arithmetic path (fp32 throughout, no bf16 rounding of
// intermediates) used for fp32 inputs and for shapes without an MFMA kernel.
//
// Math: a_ts = (q_t . k_s)^2 for s <= t (gist.science section 2.2: psi(u) = u u^T squares the
// inner product), o_t = sum a_ts v_s / (eps + sum a_ts) (section 2.1; ai.info Main Findings,
// readout-gate bullet).  Chunked form: gist.science section 2.3.
#include <algorithm>

#include "device.h"
#include "group_scores.h"
#include "phi_product.h"

namespace kata {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;   // queries (or chunk tokens) per workgroup; 4 threads per row

// ------------------------------------------------------------------------------------
// Quadratic forward.  Grid (ceil(T/64), H, B); thread (row = tid % 64, part = tid / 64)
// owns dv/4 output columns of one query.  Keys are staged 64 at a time in LDS.
// ------------------------------------------------------------------------------------
template <typename Tin, typename Tout, int P, int DV>
__global__ __launch_bounds__(kThreads) void quadratic_generic_kernel(
    DevProblem pr, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den) {
  constexpr int DP = DV / 4;
  __shared__ float ks[kRows][P];
  __shared__ float vs[kRows][DV];
  const int b = blockIdx.z, h = blockIdx.y, t0 = blockIdx.x * kRows;
  const int row = threadIdx.x % kRows, part = threadIdx.x / kRows;
  const int t = t0 + row;

  float qr[P];
  if (t < pr.T) {
    const Tin* qp = q + row_off(pr.sq, b, t, h);
#pragma unroll
    for (int i = 0; i < P; ++i) qr[i] = to_f32(qp[i]);
  } else {
#pragma unroll
    for (int i = 0; i < P; ++i) qr[i] = 0.f;
  }
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
      if (s0 + s <= t) {                       // causal mask by selection
        const float a = score_square(qr, ks[s], grp);
        l += a;
#pragma unroll
        for (int j = 0; j < DP; ++j) acc[j] = fmaf(a, vs[s][part * DP + j], acc[j]);
      }
    }
  }
  if (t < pr.T) {
    const float D = pr.eps + l;
    Tout* op = o + row_off(pr.so, b, t, h) + part * DP;
#pragma unroll
    for (int j = 0; j < DP; ++j) op[j] = from_f32<Tout>(acc[j] / D);
    if (den && part == 0) den[((long long)b * pr.T + t) * pr.H + h] = D;
  }
}

// ------------------------------------------------------------------------------------
// Chunk states, one chunk per workgroup.  Grid (n_chunks, H, B).  State layout (floats):
// e = d * p^2 + (i * p + j) for d < dv  ->  dS[i*p+j][d] = sum_s k_i k_j v_d
//     d = dv                            ->  dZ[i][j]     = sum_s k_i k_j
// ------------------------------------------------------------------------------------
template <typename Tin, int P, int DV>
__global__ __launch_bounds__(kThreads) void chunk_state_generic_kernel(
    DevProblem pr, const Tin* __restrict__ k, const Tin* __restrict__ v,
    float* __restrict__ states, int n_chunks) {
  // A (p^2 x C) . (C x (dv + 1)) product with phi(k_s) formed on the fly (phi_product).
  __shared__ __align__(16) float ks[kRows][P];
  __shared__ __align__(16) float vs[kRows][DV];
  const int b = blockIdx.z, h = blockIdx.y, c = blockIdx.x;
  const int C = pr.C, tb = c * C;
  for (int e = threadIdx.x; e < C * P; e += kThreads) {
    int s = e / P, i = e % P;
    ks[s][i] = to_f32(k[row_off(pr.sk, b, tb + s, h) + i]);
  }
  for (int e = threadIdx.x; e < C * DV; e += kThreads) {
    int s = e / DV, d = e % DV;
    vs[s][d] = to_f32(v[row_off(pr.sv, b, tb + s, h) + d]);
  }
  __syncthreads();
  constexpr int E = P * P * (DV + 1);
  phi_product<P, DV, true>(ks, vs, nullptr, C, pr.gs,
                           states + ((long long)(b * pr.H + h) * n_chunks + c) * E);
}

// ------------------------------------------------------------------------------------
// Chunk readout, one chunk per workgroup, from the exclusive prefix state S_{<c}, Z_{<c}.
// Grid (n_chunks, H, B); thread (row = token in chunk, part = dv/4 columns).  The state is
// staged in LDS, FB features at a time, as [feature][column] rows (Z in column dv), so every
// read of a wave is one broadcast; q_t's factor i comes from LDS, its factor j from registers
// (the j loop is unrolled).
// ------------------------------------------------------------------------------------
template <typename Tin, typename Tout, int P, int DV>
__global__ __launch_bounds__(kThreads) void chunk_output_generic_kernel(
    DevProblem pr, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den,
    const float* __restrict__ states, int n_chunks) {
  constexpr int PP = P * P;
  constexpr int E = PP * (DV + 1);
  constexpr int DP = DV / 4;
  constexpr int FB = 64;                         // features per staged block (FB / P rows i)
  constexpr int SROW = DV + 4;                   // floats per staged feature row (Z at DV)
  static_assert(FB % P == 0 && PP % FB == 0 && DP % 4 == 0, "readout tiling");
  __shared__ __align__(16) float ks[kRows][P];
  __shared__ __align__(16) float vs[kRows][DV];
  __shared__ float qs[kRows][P + 1];
  __shared__ __align__(16) float sl[FB][SROW];
  const int b = blockIdx.z, h = blockIdx.y, c = blockIdx.x;
  const int C = pr.C, tb = c * C;
  const int row = threadIdx.x % kRows, part = threadIdx.x / kRows;
  const bool live = row < C;
  for (int e = threadIdx.x; e < C * P; e += kThreads) {
    int s = e / P, i = e % P;
    ks[s][i] = to_f32(k[row_off(pr.sk, b, tb + s, h) + i]);
    qs[s][i] = to_f32(q[row_off(pr.sq, b, tb + s, h) + i]);
  }
  for (int e = threadIdx.x; e < C * DV; e += kThreads) {
    int s = e / DV, d = e % DV;
    vs[s][d] = to_f32(v[row_off(pr.sv, b, tb + s, h) + d]);
  }
  __syncthreads();
  const int t = tb + row;
  float qr[P];
#pragma unroll
  for (int i = 0; i < P; ++i) qr[i] = live ? qs[row][i] : 0.f;

  // inter-chunk: phi(q)^T S_{<c} and q^T Z_{<c} q, phi_f = q_i q_j
  const float* S = states + ((long long)(b * pr.H + h) * n_chunks + c) * E;
  float acc[DP];
#pragma unroll
  for (int j = 0; j < DP; ++j) acc[j] = 0.f;
  float zq = 0.f;
  StateBlock<PP, DV, FB, SROW, kThreads> nb;
  nb.load(S, 0);
  for (int f0 = 0; f0 < PP; f0 += FB) {
    __syncthreads();                             // the previous block has been read
    nb.store(sl);
    __syncthreads();
    if (f0 + FB < PP) nb.load(S, f0 + FB);       // in flight while this block is computed
    for (int ib = 0; ib < FB / P; ++ib) {
      const float qi = live ? qs[row][f0 / P + ib] : 0.f;
#pragma unroll
      for (int jj = 0; jj < P; ++jj) {
        const float phi = qi * qr[jj];
        const float* srow = sl[ib * P + jj];
#pragma unroll
        for (int j4 = 0; j4 < DP / 4; ++j4) {
          const float4 u = *reinterpret_cast<const float4*>(srow + part * DP + 4 * j4);
          acc[4 * j4] = fmaf(phi, u.x, acc[4 * j4]);
          acc[4 * j4 + 1] = fmaf(phi, u.y, acc[4 * j4 + 1]);
          acc[4 * j4 + 2] = fmaf(phi, u.z, acc[4 * j4 + 2]);
          acc[4 * j4 + 3] = fmaf(phi, u.w, acc[4 * j4 + 3]);
        }
        zq = fmaf(phi, srow[DV], zq);
      }
    }
  }
  if (!live) return;                             // no barrier follows
  // intra-chunk: causal tile, diagonal included
  float l = 0.f;
  const Groups grp = make_groups(P, pr.gs);
  for (int s = 0; s <= row; ++s) {
    const float a = score_square(qr, ks[s], grp);
    l += a;
#pragma unroll
    for (int j = 0; j < DP; ++j) acc[j] = fmaf(a, vs[s][part * DP + j], acc[j]);
  }
  const float D = pr.eps + (zq + l);
  Tout* op = o + row_off(pr.so, b, t, h) + part * DP;
#pragma unroll
  for (int j = 0; j < DP; ++j) op[j] = from_f32<Tout>(acc[j] / D);
  if (den && part == 0) den[((long long)b * pr.T + t) * pr.H + h] = D;
}

// ---- dispatch over (P, DV, dtypes) ----------------------------------------------------
template <template <typename, typename, int, int> class Launch, typename... Args>
hipError_t dispatch_io(int p, int dv, bool in_bf16, bool out_bf16, Args&&... args) {
#define KATA_CASE(P_, DV_)                                                                   \
  if (p == P_ && dv == DV_) {                                                                \
    if (in_bf16 && out_bf16) return Launch<__bf16, __bf16, P_, DV_>::run(args...);           \
    if (in_bf16) return Launch<__bf16, float, P_, DV_>::run(args...);                        \
    return Launch<float, float, P_, DV_>::run(args...);                                      \
  }
  KATA_CASE(8, 16) KATA_CASE(8, 64) KATA_CASE(16, 16) KATA_CASE(16, 64) KATA_CASE(32, 16)
  KATA_CASE(32, 64)
#undef KATA_CASE
  return hipErrorInvalidValue;
}

template <typename Tin, typename Tout, int P, int DV>
struct QuadLaunch {
  static hipError_t run(const DevProblem& pr, const void* q, const void* k, const void* v,
                        void* o, float* den, hipStream_t st) {
    dim3 grid((pr.T + kRows - 1) / kRows, pr.H, pr.B);
    launch_kernel(quadratic_generic_kernel<Tin, Tout, P, DV>, grid, kThreads, 0, st,
        pr, (const Tin*)q, (const Tin*)k, (const Tin*)v, (Tout*)o, den);
    return hipGetLastError();
  }
};

template <typename Tin, typename Tout, int P, int DV>
struct StateLaunch {
  static hipError_t run(const DevProblem& pr, const void* k, const void* v, float* states,
                        int n_chunks, hipStream_t st) {
    dim3 grid(n_chunks, pr.H, pr.B);
    launch_kernel(chunk_state_generic_kernel<Tin, P, DV>, grid, kThreads, 0, st,
        pr, (const Tin*)k, (const Tin*)v, states, n_chunks);
    return hipGetLastError();
  }
};

template <typename Tin, typename Tout, int P, int DV>
struct OutputLaunch {
  static hipError_t run(const DevProblem& pr, const void* q, const void* k, const void* v,
                        void* o, float* den, const float* states, int n_chunks,
                        hipStream_t st) {
    dim3 grid(n_chunks, pr.H, pr.B);
    launch_kernel(chunk_output_generic_kernel<Tin, Tout, P, DV>, grid, kThreads, 0, st,
        pr, (const Tin*)q, (const Tin*)k, (const Tin*)v, (Tout*)o, den, states, n_chunks);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_quadratic_generic(const DevProblem& pr, bool in_bf16, bool out_bf16,
                                    const void* q, const void* k, const void* v, void* o,
                                    float* den, hipStream_t st) {
  return dispatch_io<QuadLaunch>(pr.p, pr.dv, in_bf16, out_bf16, pr, q, k, v, o, den, st);
}

hipError_t launch_chunk_state_generic(const DevProblem& pr, bool in_bf16, const void* k,
                                      const void* v, float* states, int n_chunks,
                                      hipStream_t st) {
  // the state kernel has no output tensor; pass out_bf16 = false
  return dispatch_io<StateLaunch>(pr.p, pr.dv, in_bf16, false, pr, k, v, states, n_chunks, st);
}

hipError_t launch_chunk_output_generic(const DevProblem& pr, bool in_bf16, bool out_bf16,
                                       const void* q, const void* k, const void* v, void* o,
                                       float* den, const float* states, int n_chunks,
                                       hipStream_t st) {
  return dispatch_io<OutputLaunch>(pr.p, pr.dv, in_bf16, out_bf16, pr, q, k, v, o, den,
                                   states, n_chunks, st);
}

// Two passes over disjoint coordinate sets (p = 32 KATA-Mg as two p = 16 halves): a_ts is the
// sum of the passes' scores, so the numerators and denominators add.  Pass j left
// o_j = N_j / D_j and D_j = eps + l_j (fp32, [B][T][H][dv] and [B][T][H], contiguous):
//   o = (o_0 D_0 + o_1 D_1) / (D_0 + D_1 - eps),   D = D_0 + D_1 - eps.
// A grid-stride loop over (token, 4 value columns).
template <typename Tout>
__global__ __launch_bounds__(256) void halves_combine_kernel(
    DevProblem pr, const float* __restrict__ o0, const float* __restrict__ d0,
    const float* __restrict__ o1, const float* __restrict__ d1, Tout* __restrict__ o,
    float* __restrict__ den) {
  const int q4 = pr.dv / 4;
  const long long n = (long long)pr.B * pr.T * pr.H * q4;
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < n;
       x += (long long)gridDim.x * 256) {
    const long long tok = x / q4;
    const int c = 4 * int(x % q4);
    const int h = int(tok % pr.H), t = int((tok / pr.H) % pr.T);
    const int b = int(tok / ((long long)pr.H * pr.T));
    const float a0 = d0[tok], a1 = d1[tok], D = (a0 + a1) - pr.eps;
    const float4 u = *reinterpret_cast<const float4*>(o0 + tok * pr.dv + c);
    const float4 w = *reinterpret_cast<const float4*>(o1 + tok * pr.dv + c);
    Tout* op = o + row_off(pr.so, b, t, h) + c;
    op[0] = from_f32<Tout>(fmaf(u.x, a0, w.x * a1) / D);
    op[1] = from_f32<Tout>(fmaf(u.y, a0, w.y * a1) / D);
    op[2] = from_f32<Tout>(fmaf(u.z, a0, w.z * a1) / D);
    op[3] = from_f32<Tout>(fmaf(u.w, a0, w.w * a1) / D);
    if (den && c == 0) den[tok] = D;
  }
}

hipError_t launch_halves_combine(const DevProblem& pr, bool out_bf16, const float* o0,
                                 const float* d0, const float* o1, const float* d1, void* o,
                                 float* den, hipStream_t st) {
  if (pr.dv % 4) return hipErrorInvalidValue;
  const long long n = (long long)pr.B * pr.T * pr.H * (pr.dv / 4);
  const dim3 grid((unsigned)std::min<long long>((n + 255) / 256, 256LL * 64));
  if (out_bf16)
    launch_kernel(halves_combine_kernel<__bf16>, grid, 256, 0, st, pr, o0, d0, o1, d1,
                  (__bf16*)o, den);
  else
    launch_kernel(halves_combine_kernel<float>, grid, 256, 0, st, pr, o0, d0, o1, d1,
                  (float*)o, den);
  return hipGetLastError();
}

}  // namespace kata

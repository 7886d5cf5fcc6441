// Chunked O(T) backward of the causal normalized attention with squared scores, for gfx950.
//
// Forward (gist.science "Technische Samenvatting", sections 2.1-2.3): a_ts = (q_t . k_s)^2,
// D_t = eps + sum_{s<=t} a_ts, o_t = sum_{s<=t} a_ts v_s / D_t, computed per chunk of C tokens
// from the exclusive prefix states S_{<c} = sum vec(k k^T) v^T and Z_{<c} = sum k k^T.
// For L = sum_t <dO_t, o_t>, with g_t = dO_t / D_t and e_t = (dO_t . o_t) / D_t (derived here;
// the pages name a backward but print no formula):
//   G_ts = g_t . v_s - e_t  (s <= t),   dq_t = sum_s 2 (q_t . k_s) G_ts k_s,
//   dk_s = sum_t 2 (q_t . k_s) G_ts q_t,   dv_s = sum_{t>=s} a_ts g_t.
// Split at chunk boundaries, the part from earlier chunks of dq and from later chunks of dk,
// dv are contractions with chunk states:
//   dq_t  += 2 [mat(S_{<c} g_t) - e_t Z_{<c}] q_t
//   dk_s  += 2 [mat(R_{>c} v_s) - mat(r_{>c})] k_s,   dv_s += R_{>c}^T vec(k_s k_s^T)
// with R_{>c} = sum over later chunks of vec(q q^T) g^T and r_{>c} = sum of e vec(q q^T), a
// suffix sum that the prefix scan computes once the chunk states are stored in reverse order.
// The remaining terms are the causal tile inside each chunk.  All arithmetic is fp32: G grows
// like 1 / D_t, so no intermediate is rounded to bf16.
//
// Every kernel takes one chunk per workgroup, 256 threads = 64 rows (tokens) x 4 parts; part
// m owns the value columns [m dv/4, (m+1) dv/4) of every contraction over dv, and the partial
// p-vectors of the four parts are summed through LDS at the end.
#include <type_traits>

#include "device.h"
#include "phi_product.h"

namespace kata {
namespace {

constexpr int kRows = 64;
constexpr int kParts = 4;
constexpr int kThreads = kRows * kParts;

// g_t = dO_t / D_t (over o, in place) and e_t = (dO_t . o_t) / D_t (over D, in place).  One
// thread per token.
template <typename Tin, int DV>
__global__ __launch_bounds__(256) void bwd_chunk_prep_kernel(DevProblem pr,
                                                             const Tin* __restrict__ dO,
                                                             float* __restrict__ g,
                                                             float* __restrict__ e) {
  const long long x = (long long)blockIdx.x * 256 + threadIdx.x;   // (b * T + t) * H + h
  if (x >= (long long)pr.B * pr.T * pr.H) return;
  const int h = int(x % pr.H), t = int((x / pr.H) % pr.T), b = int(x / ((long long)pr.H * pr.T));
  const Tin* dp = dO + row_off(pr.sdo, b, t, h);
  float* gp = g + x * DV;
  const float inv = 1.f / e[x];
  float delta = 0.f;
#pragma unroll 8
  for (int d = 0; d < DV; ++d) {
    const float go = to_f32(dp[d]);
    delta = fmaf(go, gp[d], delta);
    gp[d] = go * inv;
  }
  e[x] = delta * inv;
}

// Sums the kParts partial p-vectors of each row through LDS; part 0 returns the total.
template <int P>
__device__ __forceinline__ void reduce_parts(float (&acc)[P], float (*red)[kRows][P + 1],
                                             int row, int part) {
  if (part) {
#pragma unroll
    for (int i = 0; i < P; ++i) red[part - 1][row][i] = acc[i];
  }
  __syncthreads();
  if (!part) {
#pragma unroll
    for (int m = 0; m < kParts - 1; ++m)
#pragma unroll
      for (int i = 0; i < P; ++i) acc[i] += red[m][row][i];
  }
}

// dq.  states: the forward's exclusive prefix (S_{<c}, Z_{<c}) per chunk, layout [dv+1][p^2],
// staged in LDS FB features at a time (the region is then reused for the parts' reduction).
template <typename Tin, int P, int DV>
__global__ __launch_bounds__(kThreads) void bwd_chunk_dq_kernel(
    DevProblem pr, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const float* __restrict__ g, const float* __restrict__ e,
    const float* __restrict__ states, int n_chunks, float* __restrict__ dq) {
  constexpr int PP = P * P, E = PP * (DV + 1), DP = DV / kParts;
  constexpr int FB = 32, SROW = DV + 4;
  constexpr int RED = (kParts - 1) * kRows * (P + 1), POOL = RED > FB * SROW ? RED : FB * SROW;
  static_assert(FB % P == 0, "feature blocks hold whole rows i");
  __shared__ __align__(16) float ks[kRows][P];
  __shared__ float vs[kRows][DV];
  __shared__ __align__(16) float pool[POOL];
  float (*sl)[SROW] = reinterpret_cast<float (*)[SROW]>(pool);
  float (*red)[kRows][P + 1] = reinterpret_cast<float (*)[kRows][P + 1]>(pool);
  const int b = blockIdx.z, h = blockIdx.y, c = blockIdx.x;
  const int C = pr.C, tb = c * C;
  const int row = threadIdx.x % kRows;
  const int part = __builtin_amdgcn_readfirstlane(threadIdx.x / kRows);   // one per wave
  for (int x = threadIdx.x; x < C * P; x += kThreads)
    ks[x / P][x % P] = to_f32(k[row_off(pr.sk, b, tb + x / P, h) + x % P]);
  for (int x = threadIdx.x; x < C * DV; x += kThreads)
    vs[x / DV][x % DV] = to_f32(v[row_off(pr.sv, b, tb + x / DV, h) + x % DV]);
  const bool live = row < C;
  const int t = tb + (live ? row : 0);
  float qr[P], gr[DP], acc[P];
  const Tin* qp = q + row_off(pr.sq, b, t, h);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    qr[i] = to_f32(qp[i]);
    acc[i] = 0.f;
  }
  const long long tok = ((long long)b * pr.T + t) * pr.H + h;
#pragma unroll
  for (int j = 0; j < DP; ++j) gr[j] = g[tok * DV + part * DP + j];
  const float et = e[tok];
  const float zf = part ? 0.f : -et;             // weight of the Z row: part 0 only
  // earlier chunks: u_i = sum_j q_j (sum_{d in part} S[(i,j)][d] g_d) - [part 0] e Z[i][j] q_j
  const float* S = states + ((long long)(b * pr.H + h) * n_chunks + c) * E;
  StateBlock<PP, DV, FB, SROW, kThreads> nb;
  nb.load(S, 0);
  for (int f0 = 0; f0 < PP; f0 += FB) {
    __syncthreads();                             // staging done / the previous block read
    nb.store(sl);
    __syncthreads();
    if (f0 + FB < PP) nb.load(S, f0 + FB);   // in flight while this block is computed
#pragma unroll 1
    for (int jb = 0; jb < FB; jb += P) {
      const int i = (f0 + jb) / P;
      float u = 0.f;
#pragma unroll
      for (int jj = 0; jj < P; ++jj) {
        const float* srow = sl[jb + jj];
        float m = zf * srow[DV];                 // branch-free: no wait on the loads
#pragma unroll
        for (int j4 = 0; j4 < DP / 4; ++j4) {
          const float4 u4 = *reinterpret_cast<const float4*>(srow + part * DP + 4 * j4);
          m = fmaf(u4.x, gr[4 * j4], m);
          m = fmaf(u4.y, gr[4 * j4 + 1], m);
          m = fmaf(u4.z, gr[4 * j4 + 2], m);
          m = fmaf(u4.w, gr[4 * j4 + 3], m);
        }
        u = fmaf(m, qr[jj], u);
      }
      // row i of this block (i is not a compile-time index: a select per register)
#pragma unroll
      for (int ii = 0; ii < P; ++ii) acc[ii] = ii == i ? u : acc[ii];
    }
  }
  if (live) {
    // this chunk: sum_{s<=t} (q . k_s) G_ts k_s, G_ts split over the parts' value columns
    const Groups grp = make_groups(P, pr.gs);
    // one feature group (uniform): sc[i] is the one dot product, and sc[i] * G is one product
    auto intra = [&](auto one_group) {
      for (int s = 0; s <= row; ++s) {
        float G = part ? 0.f : -et;
#pragma unroll
        for (int j = 0; j < DP; ++j) G = fmaf(gr[j], vs[s][part * DP + j], G);
        if constexpr (decltype(one_group)::value) {
          float d = 0.f;
#pragma unroll
          for (int i = 0; i < P; ++i) d = fmaf(qr[i], ks[s][i], d);
          const float dg = d * G;
#pragma unroll
          for (int i = 0; i < P; ++i) acc[i] = fmaf(dg, ks[s][i], acc[i]);
        } else {
          float sc[P];
          grouped_dots(qr, ks[s], grp, sc);
#pragma unroll
          for (int i = 0; i < P; ++i) acc[i] = fmaf(sc[i] * G, ks[s][i], acc[i]);
        }
      }
    };
    if (grp.start == 1u) intra(std::true_type{});
    else intra(std::false_type{});
  }
  __syncthreads();                               // every read of the staged state is done
  reduce_parts<P>(acc, red, row, part);
  if (live && !part) {
    float* out = dq + row_off(pr.sq, b, t, h);
#pragma unroll
    for (int i = 0; i < P; ++i) out[i] = 2.f * acc[i];
  }
}

// Per-chunk reverse states dR_c[d][f] = sum_{t in c} q_i q_j g_d (d < dv) and
// dr_c[f] = sum e_t q_i q_j (row dv), written at position n_chunks - 1 - c (phi_product).
template <typename Tin, int P, int DV>
__global__ __launch_bounds__(kThreads) void bwd_rev_state_kernel(
    DevProblem pr, const Tin* __restrict__ q, const float* __restrict__ g,
    const float* __restrict__ e, float* __restrict__ states, int n_chunks) {
  constexpr int PP = P * P, E = PP * (DV + 1);
  __shared__ __align__(16) float qs[kRows][P];
  __shared__ __align__(16) float gs[kRows][DV];
  __shared__ float es[kRows];
  const int b = blockIdx.z, h = blockIdx.y, c = blockIdx.x;
  const int C = pr.C, tb = c * C;
  for (int x = threadIdx.x; x < C * P; x += kThreads)
    qs[x / P][x % P] = to_f32(q[row_off(pr.sq, b, tb + x / P, h) + x % P]);
  for (int x = threadIdx.x; x < C * DV; x += kThreads) {
    const long long tok = ((long long)b * pr.T + tb + x / DV) * pr.H + h;
    gs[x / DV][x % DV] = g[tok * DV + x % DV];
  }
  for (int x = threadIdx.x; x < C; x += kThreads)
    es[x] = e[((long long)b * pr.T + tb + x) * pr.H + h];
  __syncthreads();
  phi_product<P, DV, false>(qs, gs, es, C, pr.gs,
                            states + ((long long)(b * pr.H + h) * n_chunks + (n_chunks - 1 - c)) * E);
}

// dk, dv.  states: R_{>c} at position n_chunks - 1 - c (the exclusive scan of the reversed
// chunk states), staged in LDS FB features at a time (the region is then reused for the
// parts' reduction).
template <typename Tin, int P, int DV>
__global__ __launch_bounds__(kThreads) void bwd_chunk_dkdv_kernel(
    DevProblem pr, const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const float* __restrict__ g, const float* __restrict__ e,
    const float* __restrict__ states, int n_chunks, float* __restrict__ dk,
    float* __restrict__ dv) {
  constexpr int PP = P * P, E = PP * (DV + 1), DP = DV / kParts;
  constexpr int FB = 32, SROW = DV + 4;
  constexpr int RED = (kParts - 1) * kRows * (P + 1), POOL = RED > FB * SROW ? RED : FB * SROW;
  static_assert(FB % P == 0, "feature blocks hold whole rows i");
  __shared__ float qs[kRows][P];
  __shared__ float ks[kRows][P + 1];              // this chunk's k rows (factor i of phi)
  __shared__ float gs[kRows][DV];
  __shared__ float es[kRows];
  __shared__ __align__(16) float pool[POOL];
  float (*rl)[SROW] = reinterpret_cast<float (*)[SROW]>(pool);
  float (*red)[kRows][P + 1] = reinterpret_cast<float (*)[kRows][P + 1]>(pool);
  const int b = blockIdx.z, h = blockIdx.y, c = blockIdx.x;
  const int C = pr.C, tb = c * C;
  const int row = threadIdx.x % kRows;
  const int part = __builtin_amdgcn_readfirstlane(threadIdx.x / kRows);   // one per wave
  for (int x = threadIdx.x; x < C * P; x += kThreads) {
    qs[x / P][x % P] = to_f32(q[row_off(pr.sq, b, tb + x / P, h) + x % P]);
    ks[x / P][x % P] = to_f32(k[row_off(pr.sk, b, tb + x / P, h) + x % P]);
  }
  for (int x = threadIdx.x; x < C * DV; x += kThreads) {
    const long long tok = ((long long)b * pr.T + tb + x / DV) * pr.H + h;
    gs[x / DV][x % DV] = g[tok * DV + x % DV];
  }
  for (int x = threadIdx.x; x < C; x += kThreads) es[x] = e[((long long)b * pr.T + tb + x) * pr.H + h];
  const bool live = row < C;
  const int s = tb + (live ? row : 0);
  float kr[P], vr[DP], acc[P], dvacc[DP];
  const Tin* kp = k + row_off(pr.sk, b, s, h);
  const Tin* vp = v + row_off(pr.sv, b, s, h) + part * DP;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    kr[i] = to_f32(kp[i]);
    acc[i] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < DP; ++j) {
    vr[j] = to_f32(vp[j]);
    dvacc[j] = 0.f;
  }
  // later chunks: w_i = sum_j k_j (sum_{d in part} R[(i,j)][d] v_d) - [part 0] r[(i,j)] k_j
  //               dv_d = sum_f R[f][d] k_i k_j   (d in part)
  const float* R = states + ((long long)(b * pr.H + h) * n_chunks + (n_chunks - 1 - c)) * E;
  const int srow_l = live ? row : 0;
  const float rf = part ? 0.f : -1.f;            // weight of the r row: part 0 only
  StateBlock<PP, DV, FB, SROW, kThreads> nb;
  nb.load(R, 0);
  for (int f0 = 0; f0 < PP; f0 += FB) {
    __syncthreads();                             // staging done / the previous block read
    nb.store(rl);
    __syncthreads();
    if (f0 + FB < PP) nb.load(R, f0 + FB);   // in flight while this block is computed
#pragma unroll 1
    for (int jb = 0; jb < FB; jb += P) {
      const int i = (f0 + jb) / P;
      const float ki = ks[srow_l][i];
      float w = 0.f;
#pragma unroll
      for (int jj = 0; jj < P; ++jj) {
        const float* rrow = rl[jb + jj];
        const float phi = ki * kr[jj];
        float m = rf * rrow[DV];                 // branch-free: no wait on the loads
#pragma unroll
        for (int j4 = 0; j4 < DP / 4; ++j4) {
          const float4 r4 = *reinterpret_cast<const float4*>(rrow + part * DP + 4 * j4);
          const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            m = fmaf(rr[y], vr[4 * j4 + y], m);
            dvacc[4 * j4 + y] = fmaf(rr[y], phi, dvacc[4 * j4 + y]);
          }
        }
        w = fmaf(m, kr[jj], w);
      }
#pragma unroll
      for (int ii = 0; ii < P; ++ii) acc[ii] = ii == i ? w : acc[ii];
    }
  }
  if (live) {
    // this chunk: t >= s
    const Groups grp = make_groups(P, pr.gs);
    // one feature group (uniform): sc[i] is the one dot product, and sc[i] * G is one product
    auto intra = [&](auto one_group) {
      for (int tt = row; tt < C; ++tt) {
        float sc[P], a, d = 0.f;
        if constexpr (decltype(one_group)::value) {
#pragma unroll
          for (int i = 0; i < P; ++i) d = fmaf(kr[i], qs[tt][i], d);
          a = fmaf(d, d, 0.f);
        } else {
          a = grouped_dots(kr, qs[tt], grp, sc);
        }
        float G = part ? 0.f : -es[tt];
#pragma unroll
        for (int j = 0; j < DP; ++j) {
          G = fmaf(gs[tt][part * DP + j], vr[j], G);
          dvacc[j] = fmaf(a, gs[tt][part * DP + j], dvacc[j]);
        }
        if constexpr (decltype(one_group)::value) {
          const float dg = d * G;
#pragma unroll
          for (int i = 0; i < P; ++i) acc[i] = fmaf(dg, qs[tt][i], acc[i]);
        } else {
#pragma unroll
          for (int i = 0; i < P; ++i) acc[i] = fmaf(sc[i] * G, qs[tt][i], acc[i]);
        }
      }
    };
    if (grp.start == 1u) intra(std::true_type{});
    else intra(std::false_type{});
    float* dvp = dv + row_off(pr.sv, b, s, h) + part * DP;
#pragma unroll
    for (int j = 0; j < DP; ++j) dvp[j] = dvacc[j];
  }
  __syncthreads();                               // every read of the staged state is done
  reduce_parts<P>(acc, red, row, part);
  if (live && !part) {
    float* out = dk + row_off(pr.sk, b, s, h);
#pragma unroll
    for (int i = 0; i < P; ++i) out[i] = 2.f * acc[i];
  }
}

template <typename Tin, int P, int DV>
struct BwdChunked {
  static hipError_t prep(const DevProblem& pr, const void* dO, float* g, float* e,
                         hipStream_t st) {
    const long long n = (long long)pr.B * pr.T * pr.H;
    launch_kernel(bwd_chunk_prep_kernel<Tin, DV>, dim3((unsigned)((n + 255) / 256)), 256, 0,
                  st, pr, (const Tin*)dO, g, e);
    return hipGetLastError();
  }
  static hipError_t dq(const DevProblem& pr, const void* q, const void* k, const void* v,
                       const float* g, const float* e, const float* states, int n_chunks,
                       float* dq, hipStream_t st) {
    launch_kernel(bwd_chunk_dq_kernel<Tin, P, DV>, dim3(n_chunks, pr.H, pr.B), kThreads, 0, st,
        pr, (const Tin*)q, (const Tin*)k, (const Tin*)v, g, e, states, n_chunks, dq);
    return hipGetLastError();
  }
  static hipError_t rev(const DevProblem& pr, const void* q, const float* g, const float* e,
                        float* states, int n_chunks, hipStream_t st) {
    launch_kernel(bwd_rev_state_kernel<Tin, P, DV>, dim3(n_chunks, pr.H, pr.B), kThreads, 0, st,
        pr, (const Tin*)q, g, e, states, n_chunks);
    return hipGetLastError();
  }
  static hipError_t dkdv(const DevProblem& pr, const void* q, const void* k, const void* v,
                         const float* g, const float* e, const float* states, int n_chunks,
                         float* dk, float* dv, hipStream_t st) {
    launch_kernel(bwd_chunk_dkdv_kernel<Tin, P, DV>, dim3(n_chunks, pr.H, pr.B), kThreads, 0, st,
        pr, (const Tin*)q, (const Tin*)k, (const Tin*)v, g, e, states, n_chunks, dk, dv);
    return hipGetLastError();
  }
};

}  // namespace

#define KATA_BWD_DISPATCH(CALL)                                                       \
  do {                                                                                \
    if (pr.C < 1 || pr.C > kRows) return hipErrorInvalidValue;                       \
    if (pr.p == 8 && pr.dv == 16) { if (in_bf16) return BwdChunked<__bf16, 8, 16>::CALL; return BwdChunked<float, 8, 16>::CALL; }     \
    if (pr.p == 8 && pr.dv == 64) { if (in_bf16) return BwdChunked<__bf16, 8, 64>::CALL; return BwdChunked<float, 8, 64>::CALL; }     \
    if (pr.p == 16 && pr.dv == 16) { if (in_bf16) return BwdChunked<__bf16, 16, 16>::CALL; return BwdChunked<float, 16, 16>::CALL; } \
    if (pr.p == 16 && pr.dv == 64) { if (in_bf16) return BwdChunked<__bf16, 16, 64>::CALL; return BwdChunked<float, 16, 64>::CALL; } \
    if (pr.p == 32 && pr.dv == 16) { if (in_bf16) return BwdChunked<__bf16, 32, 16>::CALL; return BwdChunked<float, 32, 16>::CALL; } \
    if (pr.p == 32 && pr.dv == 64) { if (in_bf16) return BwdChunked<__bf16, 32, 64>::CALL; return BwdChunked<float, 32, 64>::CALL; } \
    return hipErrorInvalidValue;                                                      \
  } while (0)

hipError_t launch_bwd_chunk_prep(const DevProblem& pr, bool in_bf16, const void* dO, float* g,
                                 float* e, hipStream_t st) {
  KATA_BWD_DISPATCH(prep(pr, dO, g, e, st));
}

hipError_t launch_bwd_chunk_dq(const DevProblem& pr, bool in_bf16, const void* q, const void* k,
                               const void* v, const float* g, const float* e,
                               const float* states, int n_chunks, float* dq, hipStream_t st) {
  KATA_BWD_DISPATCH(dq(pr, q, k, v, g, e, states, n_chunks, dq, st));
}

hipError_t launch_bwd_rev_state(const DevProblem& pr, bool in_bf16, const void* q,
                                const float* g, const float* e, float* states, int n_chunks,
                                hipStream_t st) {
  KATA_BWD_DISPATCH(rev(pr, q, g, e, states, n_chunks, st));
}

hipError_t launch_bwd_chunk_dkdv(const DevProblem& pr, bool in_bf16, const void* q,
                                 const void* k, const void* v, const float* g, const float* e,
                                 const float* states, int n_chunks, float* dk, float* dv,
                                 hipStream_t st) {
  KATA_BWD_DISPATCH(dkdv(pr, q, k, v, g, e, states, n_chunks, dk, dv, st));
}

#undef KATA_BWD_DISPATCH

}  // namespace kata

// Flash-style O(T^2) forward for gfx950 on bf16 MFMA (p = 16 with KATA-Mg group widths 16, 8,
// 4; p = 32), d_v = 64.  (gist.science "Technische Samenvatting" section 2.3: the quadratic
// operating point never forms the feature state; section 2.2: a_ts = (q_t . k_s)^2.)
//
//   o_t = sum_{s<=t} a_ts v_s / (eps + sum_{s<=t} a_ts)
//
// A workgroup of four waves takes 128 queries, each wave two 16-query tiles, and walks the
// key blocks of 64 up to its diagonal.  Per 32-key step a wave forms the squared, masked score
// tiles of both query tiles (keys as rows, so they are directly the A operands of P.V), then
// reads each V fragment once from LDS and feeds it to both query tiles: the V reads, the
// limiting LDS traffic, are spent on twice the MFMA work of one query tile per wave.  Key and
// value blocks are double-buffered in LDS (one barrier per block); the next block's global
// loads are in flight while the current one is computed.  No running maximum is kept: the
// weights are squares, so nothing needs rescaling.  The row sum of the denominator adds the
// same bf16-rounded weights that enter P.V, and runs on MFMA too (P against a block of ones).
#include "device.h"
#include "kata.h"
#include "mfma_util.h"

#include <type_traits>

namespace kata {
namespace {

constexpr int DV = 64, KB = 64;        // value width, keys per block
constexpr int QW = 32, QB = 128;       // queries per wave, per workgroup
constexpr int kThreads = 256;
constexpr int VROW = 80;               // bf16 per v row (160 B)

template <int P>
struct QTraits;
template <>
struct QTraits<16> {
  static constexpr int KROW = 20;      // bf16 per k row (40 B)
  using Frag = s16x4;
  __device__ static f32x4 mma(const Frag& a, const Frag& b) { return mfma16(a, b, zero4()); }
};
template <>
struct QTraits<32> {
  static constexpr int KROW = 40;      // bf16 per k row (80 B)
  using Frag = bf16x8;
  __device__ static f32x4 mma(const Frag& a, const Frag& b) { return mfma32(a, b, zero4()); }
};

template <int P>
struct __align__(16) QLds {
  __bf16 K[2][KB][QTraits<P>::KROW];
  __bf16 V[2][KB][VROW];
};

// score operand: row `row` of a row-major [.][ROW] bf16 tile, K-slots of lane group g
template <int P, int ROW>
__device__ __forceinline__ typename QTraits<P>::Frag score_frag(const __bf16 (*X)[ROW], int row,
                                                                 int g) {
  if constexpr (P == 16)
    return __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2*>(&X[row][4 * g]));
  else
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&X[row][8 * g]));
}

template <int P>
__device__ __forceinline__ typename QTraits<P>::Frag query_frag(const __bf16* qrow, int g,
                                                                bool live) {
  if constexpr (P == 16) {
    const uint2 u = live ? *reinterpret_cast<const uint2*>(qrow + 4 * g) : uint2{0u, 0u};
    return __builtin_bit_cast(s16x4, u);
  } else {
    const uint4 u = live ? *reinterpret_cast<const uint4*>(qrow + 8 * g) : uint4{0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, u);
  }
}

struct QStage {
  uint4 k, v0, v1;
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two fp32 -> two bf16 (round to nearest even) in one dword
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Weights of a 16-key x 16-query tile: keys s0 + 4g + r (rows), query t (this lane's column),
// squared, masked by selection where kMask (s0 + 4g + r <= t), rounded to bf16 and packed.
// GW < P (KATA-Mg, p = 16 only): one product per group of GW coordinates with the query operand
// cut to that group's lane groups, the squared group dots summed.
template <int P, int GW, bool kMask>
__device__ __forceinline__ uint2 weights(const typename QTraits<P>::Frag& kf,
                                         const typename QTraits<P>::Frag& qf, int s0, int t,
                                         int lane) {
  f32x4 x2;
  if constexpr (GW == P) {
    const f32x4 sc = QTraits<P>::mma(kf, qf);
#pragma unroll
    for (int r = 0; r < 4; ++r) x2[r] = sc[r] * sc[r];
  } else {
    static_assert(P == 16, "grouped scores at p = 16");
    const int grp = (4 * (lane >> 4)) / GW;
    x2 = zero4();
#pragma unroll
    for (int j = 0; j < P / GW; ++j) {
      const s16x4 qj = grp == j ? qf : s16x4{0, 0, 0, 0};
      const f32x4 sc = mfma16(kf, qj, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) x2[r] = fmaf(sc[r], sc[r], x2[r]);
    }
  }
  if (kMask) {
    const int s = s0 + 4 * (lane >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) x2[r] = (s + r <= t) ? x2[r] : 0.f;   // select, never multiply
  }
  return uint2{pack2(x2[0], x2[1]), pack2(x2[2], x2[3])};
}

template <typename Tout, int P, int GW>
__global__ __launch_bounds__(kThreads, 2) void quadratic_kernel(
    DevProblem pr, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den_out) {
  __shared__ QLds<P> sm;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar
  // Longest query blocks first over all (b, h) (longest-processing-time order), so short
  // sequences end without a long tail.  Consecutive blocks go to consecutive XCDs; with B*H a
  // multiple of 8 every block of one (b, h) lands on the same XCD and shares its L2 for K, V.
  const int nbh = pr.B * pr.H, id = blockIdx.x;
  const int qb = (gridDim.x / nbh) - 1 - id / nbh, h = (id % nbh) % pr.H, b = (id % nbh) / pr.H;
  const int t0 = qb * QB;
  const int tw = t0 + QW * w;                       // this wave's first query
  int tq[2];                                        // this lane's query in each query tile
  typename QTraits<P>::Frag qf[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    tq[x] = tw + 16 * x + l16;
    qf[x] = query_frag<P>(q + row_off(pr.sq, b, min(tq[x], pr.T - 1), h), g, tq[x] < pr.T);
  }

  // staging: k rows -- p = 16: threads < 128, 16 B each (row tid / 2, half tid % 2); p = 32:
  // all 256 threads (row tid / 4, quarter tid % 4); every thread 16 B of two v rows.  Loads
  // read rows clamped to T - 1 (always valid addresses); rows past T are zeroed in LDS after
  // the store, so a ragged last block carries zero keys and values.
  constexpr int KPIECES = P / 8;                    // 16-byte pieces per k row
  const bool kth = w < KB * KPIECES / 64;          // wave-uniform (w is a scalar)
  const int kr = tid / KPIECES, kc = tid % KPIECES, a2 = tid >> 3, c8 = tid & 7;
  const __bf16* kbase = k + row_off(pr.sk, b, 0, h) + 8 * kc;
  const __bf16* vbase = v + row_off(pr.sv, b, 0, h) + 8 * c8;
  const long long sk_t = pr.sk[1], sv_t = pr.sv[1];
  const int tmax = pr.T - 1;
  auto load = [&](int kb) {
    const int s0 = kb * KB, sv0 = s0 + 2 * a2;
    QStage x;
    x.k = kth ? ld16(kbase + (long long)min(s0 + kr, tmax) * sk_t) : uint4{0u, 0u, 0u, 0u};
    x.v0 = ld16(vbase + (long long)min(sv0, tmax) * sv_t);
    x.v1 = ld16(vbase + (long long)min(sv0 + 1, tmax) * sv_t);
    return x;
  };
  auto store = [&](const QStage& x, int kb) {
    const int buf = kb & 1;
    if (kth) {
      if constexpr (P == 16) {                       // 40-byte rows: two 8-byte stores
        *reinterpret_cast<uint2*>(&sm.K[buf][kr][8 * kc]) = uint2{x.k.x, x.k.y};
        *reinterpret_cast<uint2*>(&sm.K[buf][kr][8 * kc + 4]) = uint2{x.k.z, x.k.w};
      } else {
        *reinterpret_cast<uint4*>(&sm.K[buf][kr][8 * kc]) = x.k;
      }
    }
    *reinterpret_cast<uint4*>(&sm.V[buf][2 * a2][8 * c8]) = x.v0;
    *reinterpret_cast<uint4*>(&sm.V[buf][2 * a2 + 1][8 * c8]) = x.v1;
    const int s0 = kb * KB;
    if (s0 + KB > pr.T) {                            // ragged last block: zero rows >= T
      const uint4 z = {0u, 0u, 0u, 0u};
      if (kth && s0 + kr >= pr.T) {
        if constexpr (P == 16) {
          *reinterpret_cast<uint2*>(&sm.K[buf][kr][8 * kc]) = uint2{0u, 0u};
          *reinterpret_cast<uint2*>(&sm.K[buf][kr][8 * kc + 4]) = uint2{0u, 0u};
        } else {
          *reinterpret_cast<uint4*>(&sm.K[buf][kr][8 * kc]) = z;
        }
      }
      if (s0 + 2 * a2 >= pr.T) *reinterpret_cast<uint4*>(&sm.V[buf][2 * a2][8 * c8]) = z;
      if (s0 + 2 * a2 + 1 >= pr.T) *reinterpret_cast<uint4*>(&sm.V[buf][2 * a2 + 1][8 * c8]) = z;
    }
  };

  // O[x][nt]: query tile x, value columns 16 nt..; L[x]: row sums of the same bf16 weights,
  // on MFMA against a block of ones (every column holds the sum; rows are the queries)
  f32x4 O[2][4], L[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    L[x] = zero4();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) O[x][nt] = zero4();
  }
  const uint32_t one2 = 0x3F803F80u;                // two bf16 ones
  const bf16x8 ones = __builtin_bit_cast(bf16x8, uint4{one2, one2, one2, one2});

  // One 32-key step of block kb for both query tiles: weights (A operands of P.V), their row
  // sums on MFMA, then each V fragment once for both tiles.  kMask: every weight is masked by
  // selection (keys at or past the wave's first query, future keys too).
  auto step = [&](int kb, int m, auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const int buf = kb & 1, sm0 = kb * KB + 32 * m;
    bf16x8 pa[2];
#pragma unroll
    for (int x2 = 0; x2 < 2; ++x2) {
      uint2 e[2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
        e[half] = weights<P, GW, kMask>(score_frag<P>(sm.K[buf], 32 * m + 16 * half + l16, g),
                                        qf[x2], sm0 + 16 * half, tq[x2], lane);
      pa[x2] = __builtin_bit_cast(bf16x8, uint4{e[0].x, e[0].y, e[1].x, e[1].y});
      L[x2] = mfma32(pa[x2], ones, L[x2]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const bf16x8 vb = v_frag(sm.V[buf], m, nt, lane);
      O[0][nt] = mfma32(pa[0], vb, O[0][nt]);
      O[1][nt] = mfma32(pa[1], vb, O[1][nt]);
    }
  };
  using NoMask = std::integral_constant<bool, false>;
  using Mask = std::integral_constant<bool, true>;

  // Blocks [0, nf) precede every query of the workgroup (t0 is a multiple of 128): one path,
  // no masks.  Blocks [nf, last_kb] meet the diagonal of some wave.
  const int last_kb = min((t0 + QB - 1) / KB, (pr.T - 1) / KB);
  const int nf = t0 / KB;
  QStage x = load(0);
  store(x, 0);
  x = load(min(1, last_kb));
  __syncthreads();
  for (int kb = 0; kb < nf; ++kb) {
    step(kb, 0, NoMask{});
    step(kb, 1, NoMask{});
    store(x, kb + 1);                                // kb + 1 <= nf <= last_kb; its buffer
    x = load(min(kb + 2, last_kb));                  // was read before the last barrier
    __syncthreads();
  }
  for (int kb = nf; kb <= last_kb; ++kb) {
    const int s_base = kb * KB;
    if (s_base + KB - 1 < tw) {                     // the whole block precedes the wave's queries
      step(kb, 0, NoMask{});
      step(kb, 1, NoMask{});
    } else if (s_base < tw + QW) {                  // the block meets the wave's diagonal
      step(kb, 0, Mask{});
      if (s_base + 32 < tw + QW) step(kb, 1, Mask{});
    }
    if (kb + 1 <= last_kb) {
      store(x, kb + 1);
      x = load(min(kb + 2, last_kb));
    }
    __syncthreads();
  }

  // gated outputs: lane holds queries tw + 16 x + 4g + r (rows), columns 16 nt + l16
#pragma unroll
  for (int x2 = 0; x2 < 2; ++x2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = tw + 16 * x2 + 4 * g + r;
      const float D = pr.eps + L[x2][r];
      if (tr >= pr.T) continue;
      const float ir = 1.f / D;
      Tout* op = o + row_off(pr.so, b, tr, h);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) op[16 * nt + l16] = cvt_out<Tout>(O[x2][nt][r] * ir);
      if (den_out && l16 == 0) den_out[((long long)b * pr.T + tr) * pr.H + h] = D;
    }
  }
}

template <typename Tout, int P, int GW>
void launch_t(const DevProblem& pr, hipStream_t st, const void* q, const void* k,
              const void* v, void* o, float* den) {
  dim3 grid(((pr.T + QB - 1) / QB) * pr.H * pr.B);
  quadratic_kernel<Tout, P, GW><<<grid, kThreads, 0, st>>>(
      pr, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (Tout*)o, den);
}

template <typename Tout>
hipError_t launch_dispatch(const DevProblem& pr, int gw, hipStream_t st, const void* q,
                           const void* k, const void* v, void* o, float* den) {
  if (pr.p == 16 && gw == 16) launch_t<Tout, 16, 16>(pr, st, q, k, v, o, den);
  else if (pr.p == 16 && gw == 8) launch_t<Tout, 16, 8>(pr, st, q, k, v, o, den);
  else if (pr.p == 16 && gw == 4) launch_t<Tout, 16, 4>(pr, st, q, k, v, o, den);
  else if (pr.p == 32 && gw == 32) launch_t<Tout, 32, 32>(pr, st, q, k, v, o, den);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

// The grid is one-dimensional: every query block of every (b, h).
bool quadratic_mfma_grid_fits(const DevProblem& pr) {
  return int64_t((pr.T + QB - 1) / QB) * pr.B * pr.H <= 0x7fffffffLL;
}

// gw: KATA-Mg group width (p for a single group)
hipError_t launch_quadratic_mfma(const DevProblem& pr, int gw, bool out_bf16, const void* q,
                                 const void* k, const void* v, void* o, float* den,
                                 hipStream_t st) {
  if (pr.dv != DV || !quadratic_mfma_grid_fits(pr)) return hipErrorInvalidValue;
  return out_bf16 ? launch_dispatch<__bf16>(pr, gw, st, q, k, v, o, den)
                  : launch_dispatch<float>(pr, gw, st, q, k, v, o, den);
}

}  // namespace kata

// Flash-style O(T^2) forward for gfx950 on bf16 MFMA (p = 16 with KATA-Mg group widths 16, 8,
// 4; p = 32 with group widths 32, 16, 8, 4), d_v = 64.  (gist.science "Technische
// Samenvatting" section 2.3: the quadratic operating point never forms the feature state;
// section 2.2: a_ts = (q_t . k_s)^2.)
//
//   o_t = sum_{s<=t} a_ts v_s / (eps + sum_{s<=t} a_ts)
//
// A workgroup of four waves takes 4 QW queries; a wave holds NB blocks of 32 queries and walks
// the key blocks of 64 up to its diagonal, 32 keys per step.  Every product is the full-rate
// 32x32x16 bf16 MFMA (the 16-deep 16x16 shape runs at half rate on gfx950):
//   scores  S^T (32 keys x 32 queries) = K_step . Q^T, depth p (one product at p = 16, two at
//           p = 32; KATA-Mg: one per group with the query operand cut to the group);
//   P.V     O (32 queries x 64 values) += P (32 x 32 keys) . V_step, four products.
// The result layout of the score product (lane l: query l % 32, keys 8 (v / 4) + 4 (l / 32) +
// v % 4 for its 16 registers v) is, after squaring and rounding to bf16, directly the A operand
// of P.V for two 16-key halves; the V operands are read in that key order with LDS transpose
// loads, once per step for all NB query blocks of the wave.  The denominator's row sums add the
// same bf16-rounded weights that enter P.V (dot2 against ones, fp32 accumulate).  No running
// maximum is kept: the weights are squares, so nothing needs rescaling.  Key and value blocks
// are double-buffered in LDS (one barrier per block); the next block's global loads are in
// flight while the current one is computed.
#include "device.h"
#include "kata.h"
#include "mfma_util.h"

#include <type_traits>

namespace kata {
namespace {

constexpr int DV = 64, KB = 64;        // value width, keys per block
constexpr int kThreads = 256;          // four waves
constexpr int VROW = 80;               // bf16 per v row (160 B: transpose reads conflict-free)

// NB blocks of 32 queries per wave
template <int NB>
struct QShape {
  static constexpr int QW = 32 * NB, QB = 4 * QW;
};

template <int P>
struct QTraits;
template <>
struct QTraits<16> {
  static constexpr int KROW = 24;      // bf16 per k row (48 B, 16-byte aligned pieces)
  static constexpr int KD = 1;         // 16-deep products per score block
};
template <>
struct QTraits<32> {
  static constexpr int KROW = 40;      // 80 B
  static constexpr int KD = 2;
};

template <int P>
struct __align__(16) QLds {
  __bf16 K[2][KB][QTraits<P>::KROW];
  __bf16 V[2][KB][VROW];
};

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma3232(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// row of result register v of a 32x32 product in lane half h (= lane / 32)
__device__ __forceinline__ int row_of(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// two fp32 -> two bf16 (round to nearest even) in one dword
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// running fp32 sum of the two bf16 in w
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
}

// Query operand of one 16-deep K step cut to KATA-Mg group j of width GW (8 or 4) within the
// step: lane half h holds the step's coordinates 8h .. 8h + 7.
template <int GW>
__device__ __forceinline__ bf16x8 group_cut(const bf16x8& q, int h, int j) {
  const uint4 u = __builtin_bit_cast(uint4, q);
  uint4 r = {0u, 0u, 0u, 0u};
  if constexpr (GW == 8) {
    if (h == j) r = u;
  } else {                                          // GW == 4: coordinates 8h + 4x .. + 3
    if (2 * h == j) r = uint4{u.x, u.y, 0u, 0u};
    if (2 * h + 1 == j) r = uint4{0u, 0u, u.z, u.w};
  }
  return __builtin_bit_cast(bf16x8, r);
}

// Squared scores x2 of a 32-key x 32-query block (keys s0 + row_of(v, h), query t) -> the
// packed bf16 A operand of P.V, masked by selection where kMask; lsum adds the rounded values.
template <bool kMask>
__device__ __forceinline__ void pack_weights(f32x16 x2, int s0, int t, int h, uint32_t (&pw)[8],
                                             float& lsum) {
  if (kMask) {
#pragma unroll
    for (int v = 0; v < 16; ++v) x2[v] = (s0 + row_of(v, h) <= t) ? x2[v] : 0.f;   // select
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pw[j] = pack2(x2[2 * j], x2[2 * j + 1]);
    lsum = add_pair(pw[j], lsum);
  }
}

// Weights of a 32-key x 32-query block as the packed bf16 A operand of P.V: keys s0 +
// row_of(v, h) against query t (this lane's), squared (GW < P: squared group dots summed),
// masked by selection where kMask, rounded to bf16; lsum adds the rounded values.
template <int P, int GW, bool kMask>
__device__ __forceinline__ void weights(const bf16x8 (&kf)[QTraits<P>::KD],
                                        const bf16x8 (&qf)[QTraits<P>::KD], int s0, int t,
                                        int h, uint32_t (&pw)[8], float& lsum) {
  f32x16 x2;
  if constexpr (GW == P) {
    f32x16 sc = mfma3232(kf[0], qf[0], zero16());
    if constexpr (QTraits<P>::KD == 2) sc = mfma3232(kf[1], qf[1], sc);
#pragma unroll
    for (int v = 0; v < 16; ++v) x2[v] = sc[v] * sc[v];
  } else {
    // one product per group: a 16-deep K step holds 16 / GW groups (GW = 16: the whole step)
    static_assert(GW == 16 || GW == 8 || GW == 4, "group widths 16, 8, 4");
    x2 = zero16();
#pragma unroll
    for (int d = 0; d < QTraits<P>::KD; ++d)
#pragma unroll
      for (int j = 0; j < 16 / GW; ++j) {
        bf16x8 qg = qf[d];
        if constexpr (GW < 16) qg = group_cut<GW>(qf[d], h, j);
        const f32x16 sc = mfma3232(kf[d], qg, zero16());
#pragma unroll
        for (int v = 0; v < 16; ++v) x2[v] = fmaf(sc[v], sc[v], x2[v]);
      }
  }
  pack_weights<kMask>(x2, s0, t, h, pw, lsum);
}

// V operand of P.V for keys [kb0, kb0 + 16) in score row order and value columns [c0, c0 + 32):
// lane l needs V[kb0 + row_of(i, h)][c0 + l % 32] in slot i.  Two LDS transpose loads (slots
// 0-3: keys kb0 + 4h + 0..3, slots 4-7: 8 further); within a 16-lane block, lane j points at
// V[row + j / 4][col + 4 (j % 4)], which hands lane i the value V[row + r][col + i] in slot r.
__device__ __forceinline__ bf16x8 v_frag32(const __bf16 (*V)[VROW], int kb0, int c0, int lane) {
  const int h = lane >> 5, j = lane & 15;
  const int row = kb0 + 4 * h + (j >> 2), col = c0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&V[row][col]));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&V[row + 8][col]));
  const uint2 ul = __builtin_bit_cast(uint2, lo), uh = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, uint4{ul.x, ul.y, uh.x, uh.y});
}

struct QStage {
  uint4 k, v0, v1;
};

// ---- non-finite values: the exact path of a wave ---------------------------------------
// In a masked step the P.V product still multiplies a masked weight P_ts = 0 with the value
// v_s of every key of the step, and 0 * inf or 0 * nan is nan: a non-finite value of a later
// token would reach earlier outputs of its key block.  The kernel therefore checks the wave's
// accumulators before the gate; when one is non-finite (a non-finite input, a rare case), the
// wave evaluates its outputs again here: the same products in the same order per
// accumulator, operands read from global memory, and in masked steps value operands with their
// non-finite entries replaced by zero (masked pairs then add exact zeros, as they do for
// finite values) plus the exact contributions of the non-finite values of unmasked pairs,
// pair by pair.  Outputs that see no non-finite value are bitwise those of the main path.

// One head's rows in global memory for the exact path: base pointers at token 0 and element
// strides between consecutive tokens.
struct HeadRows {
  const __bf16 *q, *k, *v;
  long long sq, sk, sv;
  int T;
};

// K operand of key step m of block kb from global memory (the LDS tile's values; keys past T
// are zero rows): key kb * KB + 32 m + lane % 32, coordinates 16 d + 8 (lane / 32) ..
__device__ __forceinline__ bf16x8 k_frag_global(const HeadRows& hr, int kb, int m, int d,
                                                int lane) {
  const int s = kb * KB + 32 * m + (lane & 31);
  const uint4 u = s < hr.T ? ld16(hr.k + s * hr.sk + 16 * d + 8 * (lane >> 5))
                           : uint4{0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, u);
}

// V operand of P.V from global memory, the layout of v_frag32: keys kb0 + row_of(i, lane / 32)
// in slot i, value column c0 + lane % 32 (keys past T are zero rows)
__device__ __forceinline__ bf16x8 v_frag_global(const HeadRows& hr, int kb0, int c0, int lane) {
  const int h = lane >> 5, l32 = lane & 31;
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int s = kb0 + 8 * (i >> 2) + 4 * h + (i & 3);
    f[i] = s < hr.T ? hr.v[s * hr.sv + c0 + l32] : (__bf16)0.f;
  }
  return f;
}

// O[n][vr] (query t0 + row_of(vr, lane / 32), value column 32 n + lane % 32) += P * V for every
// key s of [s0, s0 + 32) up to that query whose value is non-finite; pw: this lane's packed
// weights of the step (query t0 + lane % 32, keys s0 + row_of(v, h) in register v), handed to
// the other lanes by shuffles.
__device__ __forceinline__ void nonfinite_terms32(f32x16 (&O)[2], const HeadRows& hr,
                                                  const uint32_t (&pw)[8], int s0, int t0,
                                                  int lane) {
  const int h = lane >> 5, l32 = lane & 31;
  for (int j = 0; j < 32; ++j) {
    const int s = s0 + j;
    if (s > t0 + 31 || s >= hr.T) break;             // uniform
    // the weight of (query row r, key j) sits in lane 32 ((j / 4) % 2) + r, register
    // 4 (j / 8) + j % 4, i.e. half (j % 2) of packed word 2 (j / 8) + (j % 4) / 2
    const int word = 2 * (j >> 3) + ((j & 3) >> 1);
    uint32_t d = pw[0];
#pragma unroll
    for (int x = 1; x < 8; ++x) d = word == x ? pw[x] : d;
    const int src = 32 * ((j >> 2) & 1);
    const __bf16 x0 = hr.v[s * hr.sv + l32], x1 = hr.v[s * hr.sv + 32 + l32];
    const bool b0 = nonfinite_bf16(x0), b1 = nonfinite_bf16(x1);
    const float f0 = (float)x0, f1 = (float)x1;
#pragma unroll
    for (int vr = 0; vr < 16; ++vr) {
      const int row = row_of(vr, h);
      const uint32_t wd = (uint32_t)__shfl((int)d, src + row);
      const float wgt = (j & 1) ? bf_hi(wd) : bf_lo(wd);
      if (s <= t0 + row) {
        if (b0) O[0][vr] += wgt * f0;
        if (b1) O[1][vr] += wgt * f1;
      }
    }
  }
}

// The exact path of one wave (see above): its NB query blocks from tw on, evaluated again
// (accumulators and row sums, each in the main path's order) and stored over the outputs the
// main path wrote (o: the head's output row of token 0, so: the token stride; D_t is unchanged).
// Called after the main path's stores, when little else is live, with a few scalar arguments;
// not inlined, so the main loops keep their registers.
template <typename Tout, int P, int GW, int NB>
__device__ __attribute__((noinline)) void quadratic_wave_exact(
    const __bf16* qh, const __bf16* kh, const __bf16* vh, Tout* oh, long long sq, long long sk,
    long long sv, long long so, int T, float eps, int tw, int lane) {
  constexpr int QW = QShape<NB>::QW, KD = QTraits<P>::KD;
  const HeadRows hr{qh, kh, vh, sq, sk, sv, T};
  const int h = lane >> 5, l32 = lane & 31;
  bf16x8 qf[NB][KD];
  int tq[NB];
  f32x16 O[NB][2];
  float lsum[NB];
#pragma unroll
  for (int x = 0; x < NB; ++x) {
    tq[x] = tw + 32 * x + l32;
    const __bf16* qrow = qh + min(tq[x], T - 1) * sq;
#pragma unroll
    for (int d = 0; d < KD; ++d)
      qf[x][d] = __builtin_bit_cast(bf16x8, tq[x] < T ? ld16(qrow + 16 * d + 8 * h)
                                                      : uint4{0u, 0u, 0u, 0u});
    O[x][0] = O[x][1] = zero16();
    lsum[x] = 0.f;
  }
  const int last_kb = min((tw + QW - 1) / KB, (T - 1) / KB);
  for (int kb = 0; kb <= last_kb; ++kb) {
    const int s_base = kb * KB;
    const bool full = s_base + KB - 1 < tw;
    const int n_steps = full ? 2 : (s_base + 32 < tw + QW ? 2 : 1);
    for (int m = 0; m < n_steps; ++m) {
      const int sm0 = s_base + 32 * m;
      bf16x8 kf[KD];
#pragma unroll
      for (int d = 0; d < KD; ++d) kf[d] = k_frag_global(hr, kb, m, d, lane);
      uint32_t pw[NB][8];
      bool live[NB];
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        live[x] = full || sm0 <= tw + 32 * x + 31;
        if (!live[x]) continue;
        if (full) weights<P, GW, false>(kf, qf[x], sm0, tq[x], h, pw[x], lsum[x]);
        else weights<P, GW, true>(kf, qf[x], sm0, tq[x], h, pw[x], lsum[x]);
      }
#pragma unroll
      for (int kh2 = 0; kh2 < 2; ++kh2)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          bf16x8 vb = v_frag_global(hr, sm0 + 16 * kh2, 32 * n, lane);
          if (!full) vb = finite_or_zero(vb);
#pragma unroll
          for (int x = 0; x < NB; ++x) {
            if (!live[x]) continue;
            const bf16x8 pa = __builtin_bit_cast(
                bf16x8, uint4{pw[x][4 * kh2], pw[x][4 * kh2 + 1], pw[x][4 * kh2 + 2], pw[x][4 * kh2 + 3]});
            O[x][n] = mfma3232(pa, vb, O[x][n]);
          }
        }
      if (!full) {
#pragma unroll
        for (int x = 0; x < NB; ++x)
          if (live[x]) nonfinite_terms32(O[x], hr, pw[x], sm0, tw + 32 * x, lane);
      }
    }
  }
#pragma unroll
  for (int xb = 0; xb < NB; ++xb) {
    const float lq = lsum[xb] + __shfl_xor(lsum[xb], 32);
#pragma unroll
    for (int vr = 0; vr < 16; ++vr) {
      const int row = row_of(vr, h), tr = tw + 32 * xb + row;
      const float D = eps + __shfl(lq, row);
      if (tr >= T) continue;
      const float ir = 1.f / D;
      Tout* op = oh + tr * so;
      op[l32] = from_f32<Tout>(O[xb][0][vr] * ir);
      op[32 + l32] = from_f32<Tout>(O[xb][1][vr] * ir);
    }
  }
}

template <typename Tout, int P, int GW, int NB>
__global__ __launch_bounds__(kThreads, NB == 1 ? 3 : 2) void quadratic_kernel(
    DevProblem pr, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den_out) {
  constexpr int QW = QShape<NB>::QW, QB = QShape<NB>::QB, KD = QTraits<P>::KD;
  __shared__ QLds<P> sm;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar
  // Longest query blocks first over all (b, h) (longest-processing-time order), so short
  // sequences end without a long tail.  Consecutive blocks go to consecutive XCDs; with B*H a
  // multiple of 8 every block of one (b, h) lands on the same XCD and shares its L2 for K, V.
  const int nbh = pr.B * pr.H, id = blockIdx.x;
  const int qb = (gridDim.x / nbh) - 1 - id / nbh, hd = (id % nbh) % pr.H, b = (id % nbh) / pr.H;
  const int t0 = qb * QB;
  const int tw = t0 + QW * w;                       // this wave's first query
  int tq[NB];                                       // this lane's query in each query block
  bf16x8 qf[NB][KD];                                // Q^T operands: coordinates 16 d + 8 h + i
#pragma unroll
  for (int x = 0; x < NB; ++x) {
    tq[x] = tw + 32 * x + l32;
    const __bf16* qrow = q + row_off(pr.sq, b, min(tq[x], pr.T - 1), hd);
#pragma unroll
    for (int d = 0; d < KD; ++d) {
      const uint4 u = tq[x] < pr.T ? ld16(qrow + 16 * d + 8 * h) : uint4{0u, 0u, 0u, 0u};
      qf[x][d] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // staging: k rows -- p = 16: threads < 128, 16 B each (row tid / 2, half tid % 2); p = 32:
  // all 256 threads (row tid / 4, quarter tid % 4); every thread 16 B of two v rows.  Loads
  // read rows clamped to T - 1 (always valid addresses); rows past T are zeroed in LDS after
  // the store, so a ragged last block carries zero keys and values.
  constexpr int KPIECES = P / 8;                    // 16-byte pieces per k row
  const bool kth = w < KB * KPIECES / 64;          // wave-uniform (w is a scalar)
  const int kr = tid / KPIECES, kc = tid % KPIECES, a2 = tid >> 3, c8 = tid & 7;
  const __bf16* kbase = k + row_off(pr.sk, b, 0, hd) + 8 * kc;
  const __bf16* vbase = v + row_off(pr.sv, b, 0, hd) + 8 * c8;
  const long long sk_t = pr.sk[1], sv_t = pr.sv[1];
  const int tmax = pr.T - 1;
  // this thread's rows within a block (fixed); the block offset s0 * stride is wave-uniform
  const __bf16* krow = kbase + (long long)kr * sk_t;
  const __bf16* vrow = vbase + (long long)(2 * a2) * sv_t;
  auto load = [&](int kb) {
    const int s0 = kb * KB;
    QStage x;
    if (s0 + KB <= pr.T) {                          // whole block in range
      const __bf16* vp = vrow + (long long)s0 * sv_t;
      x.k = kth ? ld16(krow + (long long)s0 * sk_t) : uint4{0u, 0u, 0u, 0u};
      x.v0 = ld16(vp);
      x.v1 = ld16(vp + sv_t);
    } else {                                        // ragged last block: rows clamped to T - 1
      const int sv0 = s0 + 2 * a2;
      x.k = kth ? ld16(kbase + (long long)min(s0 + kr, tmax) * sk_t) : uint4{0u, 0u, 0u, 0u};
      x.v0 = ld16(vbase + (long long)min(sv0, tmax) * sv_t);
      x.v1 = ld16(vbase + (long long)min(sv0 + 1, tmax) * sv_t);
    }
    return x;
  };
  auto store = [&](const QStage& x, int kb) {
    const int buf = kb & 1;
    if (kth) *reinterpret_cast<uint4*>(&sm.K[buf][kr][8 * kc]) = x.k;
    *reinterpret_cast<uint4*>(&sm.V[buf][2 * a2][8 * c8]) = x.v0;
    *reinterpret_cast<uint4*>(&sm.V[buf][2 * a2 + 1][8 * c8]) = x.v1;
    const int s0 = kb * KB;
    if (s0 + KB > pr.T) {                            // ragged last block: zero rows >= T
      const uint4 z = {0u, 0u, 0u, 0u};
      if (kth && s0 + kr >= pr.T) *reinterpret_cast<uint4*>(&sm.K[buf][kr][8 * kc]) = z;
      if (s0 + 2 * a2 >= pr.T) *reinterpret_cast<uint4*>(&sm.V[buf][2 * a2][8 * c8]) = z;
      if (s0 + 2 * a2 + 1 >= pr.T) *reinterpret_cast<uint4*>(&sm.V[buf][2 * a2 + 1][8 * c8]) = z;
    }
  };

  // O[x][n]: query block x, value columns 32 n ..; lsum[x]: this lane's share (its 16 keys of
  // each step) of the row sum of query tq[x]
  f32x16 O[NB][2];
  float lsum[NB];
#pragma unroll
  for (int x = 0; x < NB; ++x) {
    lsum[x] = 0.f;
    O[x][0] = zero16();
    O[x][1] = zero16();
  }

  // One 32-key step m of block kb for the wave's query blocks.  kMask: every weight is masked
  // by selection, and query blocks wholly before the step's keys are skipped.
  auto step = [&](int kb, int m, auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const int buf = kb & 1, sm0 = kb * KB + 32 * m;
    bf16x8 kf[KD];                                  // K operand: key 32 m + l32, coords 16 d + 8 h
#pragma unroll
    for (int d = 0; d < KD; ++d)
      kf[d] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                             &sm.K[buf][32 * m + l32][16 * d + 8 * h]));
    uint32_t pw[NB][8];
    bool live[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      live[x] = !kMask || sm0 <= tw + 32 * x + 31;  // wave-uniform
      if (live[x]) weights<P, GW, kMask>(kf, qf[x], sm0, tq[x], h, pw[x], lsum[x]);
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const bf16x8 vb = v_frag32(sm.V[buf], 32 * m + 16 * kh, 32 * n, lane);
#pragma unroll
        for (int x = 0; x < NB; ++x) {
          if (!live[x]) continue;
          const bf16x8 pa = __builtin_bit_cast(
              bf16x8, uint4{pw[x][4 * kh], pw[x][4 * kh + 1], pw[x][4 * kh + 2], pw[x][4 * kh + 3]});
          O[x][n] = mfma3232(pa, vb, O[x][n]);
        }
      }
    }
  };
  using NoMask = std::integral_constant<bool, false>;
  using Mask = std::integral_constant<bool, true>;

  // A whole unmasked block (single feature group): every score product of the block first, so
  // that the weights of one query block (VALU) run beside the P.V products of the previous one.
  auto block_nomask = [&](int kb) {
    const int buf = kb & 1;
    f32x16 sc[2][NB];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8 kf[KD];
#pragma unroll
      for (int d = 0; d < KD; ++d)
        kf[d] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                               &sm.K[buf][32 * m + l32][16 * d + 8 * h]));
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        sc[m][x] = mfma3232(kf[0], qf[x][0], zero16());
        if constexpr (KD == 2) sc[m][x] = mfma3232(kf[1], qf[x][1], sc[m][x]);
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8 vb[2][2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int n = 0; n < 2; ++n) vb[kh][n] = v_frag32(sm.V[buf], 32 * m + 16 * kh, 32 * n, lane);
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        f32x16 x2;
#pragma unroll
        for (int r = 0; r < 16; ++r) x2[r] = sc[m][x][r] * sc[m][x][r];
        uint32_t pw[8];
        pack_weights<false>(x2, 0, 0, h, pw, lsum[x]);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const bf16x8 pa = __builtin_bit_cast(
              bf16x8, uint4{pw[4 * kh], pw[4 * kh + 1], pw[4 * kh + 2], pw[4 * kh + 3]});
#pragma unroll
          for (int n = 0; n < 2; ++n) O[x][n] = mfma3232(pa, vb[kh][n], O[x][n]);
        }
      }
    }
  };
  auto full_block = [&](int kb) {
    if constexpr (GW == P) {
      block_nomask(kb);
    } else {
      step(kb, 0, NoMask{});
      step(kb, 1, NoMask{});
    }
  };

  // Blocks [0, nf) precede every query of the workgroup (t0 is a multiple of 64): one path,
  // no masks.  Blocks [nf, last_kb] meet the diagonal of some wave.
  const int last_kb = min((t0 + QB - 1) / KB, (pr.T - 1) / KB);
  const int nf = t0 / KB;
  QStage x = load(0);
  store(x, 0);
  x = load(min(1, last_kb));
  __syncthreads();
  for (int kb = 0; kb < nf; ++kb) {
    full_block(kb);
    store(x, kb + 1);                                // kb + 1 <= nf <= last_kb; its buffer
    x = load(min(kb + 2, last_kb));                  // was read before the last barrier
    __syncthreads();
  }
  for (int kb = nf; kb <= last_kb; ++kb) {
    const int s_base = kb * KB;
    if (s_base + KB - 1 < tw) {                     // the whole block precedes the wave's queries
      full_block(kb);
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

  // gated outputs: register v of O[x][n] holds query tw + 32 x + row_of(v, h), column
  // 32 n + l32; the full row sum of query i of a block is lsum in lanes i and i + 32
  bool bad = false;
#pragma unroll
  for (int xb = 0; xb < NB; ++xb) {
    const float lq = lsum[xb] + __shfl_xor(lsum[xb], 32);
#pragma unroll
    for (int vr = 0; vr < 16; ++vr) {
      const int row = row_of(vr, h), tr = tw + 32 * xb + row;
      const float D = pr.eps + __shfl(lq, row);
      if (tr >= pr.T) continue;
      const float ir = 1.f / D;
      Tout* op = o + row_off(pr.so, b, tr, hd);
      const float o0 = O[xb][0][vr] * ir, o1 = O[xb][1][vr] * ir;
      bad |= !__builtin_isfinite(o0) || !__builtin_isfinite(o1);
      op[l32] = from_f32<Tout>(o0);
      op[32 + l32] = from_f32<Tout>(o1);
      if (den_out && l32 == 0) den_out[((long long)b * pr.T + tr) * pr.H + hd] = D;
    }
  }
  // a non-finite output (a non-finite input: rare): the wave's exact path over it
  if (__any(bad))
    quadratic_wave_exact<Tout, P, GW, NB>(
        q + row_off(pr.sq, b, 0, hd), k + row_off(pr.sk, b, 0, hd), v + row_off(pr.sv, b, 0, hd),
        o + row_off(pr.so, b, 0, hd), pr.sq[1], pr.sk[1], pr.sv[1], pr.so[1], pr.T, pr.eps, tw,
        lane);
}

// query blocks of 32 per wave: two where the grid still holds several waves of workgroups
// (each V operand then feeds two products), one for short sequences
int blocks_per_wave(const DevProblem& pr) {
  const long long wg2 = (long long)((pr.T + QShape<2>::QB - 1) / QShape<2>::QB) * pr.B * pr.H;
  return wg2 >= 4096 ? 2 : 1;
}

template <typename Tout, int P, int GW>
void launch_t(const DevProblem& pr, hipStream_t st, const void* q, const void* k,
              const void* v, void* o, float* den) {
  auto go = [&](auto nb_tag) {
    constexpr int NB = decltype(nb_tag)::value, QB = QShape<NB>::QB;
    dim3 grid(((pr.T + QB - 1) / QB) * pr.H * pr.B);
    launch_kernel(quadratic_kernel<Tout, P, GW, NB>, grid, kThreads, 0, st,
        pr, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (Tout*)o, den);
  };
  if (blocks_per_wave(pr) == 2) go(std::integral_constant<int, 2>{});
  else go(std::integral_constant<int, 1>{});
}

template <typename Tout>
hipError_t launch_dispatch(const DevProblem& pr, int gw, hipStream_t st, const void* q,
                           const void* k, const void* v, void* o, float* den) {
  if (pr.p == 16 && gw == 16) launch_t<Tout, 16, 16>(pr, st, q, k, v, o, den);
  else if (pr.p == 16 && gw == 8) launch_t<Tout, 16, 8>(pr, st, q, k, v, o, den);
  else if (pr.p == 16 && gw == 4) launch_t<Tout, 16, 4>(pr, st, q, k, v, o, den);
  else if (pr.p == 32 && gw == 32) launch_t<Tout, 32, 32>(pr, st, q, k, v, o, den);
  else if (pr.p == 32 && gw == 16) launch_t<Tout, 32, 16>(pr, st, q, k, v, o, den);
  else if (pr.p == 32 && gw == 8) launch_t<Tout, 32, 8>(pr, st, q, k, v, o, den);
  else if (pr.p == 32 && gw == 4) launch_t<Tout, 32, 4>(pr, st, q, k, v, o, den);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

// KATA-Mg group width the MFMA kernel takes for this problem (bf16 in, d_v = 64, p = 16 or
// 32, groups of 16, 8 or 4 coordinates, or the whole p), 0 when it takes none.
int quadratic_mfma_group_width(const kata_problem* pr) {
  if (pr->in_dtype != KATA_BF16 || pr->dv != DV || (pr->p != 16 && pr->p != 32)) return 0;
  const int g = pr->groups <= 1 ? 1 : pr->groups;
  if (pr->p % g) return 0;
  const int gw = pr->p / g;
  return (gw == pr->p || gw == 16 || gw == 8 || gw == 4) ? gw : 0;
}

// The grid is one-dimensional: every query block of every (b, h).
bool quadratic_mfma_grid_fits(const DevProblem& pr) {
  constexpr int QB = QShape<1>::QB;                 // the smaller block: the larger grid
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

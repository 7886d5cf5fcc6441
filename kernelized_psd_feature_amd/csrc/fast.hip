// bf16 MFMA kernels for gfx950 (p = 16, d_v = 64, chunk C = 64): the chunk-state build, the
// segment walk of the chunked forward (intra-chunk tile + inter-chunk readout + output gate +
// state update), and the flash-style quadratic forward.
//
// Method (gist.science "Technische Samenvatting" sections 2.1-2.3; ai.info AI summary, Main
// Findings): a_ts = (q_t . k_s)^2 = <vec(q q^T), vec(k k^T)>, o_t = sum_{s<=t} a_ts v_s / D_t,
// D_t = eps + sum_{s<=t} a_ts.  Chunked form: the state S = sum vec(k k^T) v^T (p^2 x d_v) and
// Z = sum k k^T are summed per chunk, prefix-scanned over chunks, and read out with
// vec(q q^T); inside a chunk the causal tile is evaluated directly.
//
// Precision (fixed here, the pages leave it open): every product runs on bf16 MFMA with fp32
// accumulation.  The squared scores P are rounded to bf16 for the P.V product and the row sum
// of the denominator is taken from the same rounded values, so each output stays an exact
// convex combination of the values it mixes.  Feature products k_i k_j and q_i q_j are formed
// in fp32 and rounded to bf16; the running state S is fp32 in registers and rounded to bf16
// only as a readout operand.  Z = sum k k^T is exact (bf16 x bf16 products in fp32), and the
// inter-chunk denominator q^T Z q is evaluated in fp32 on the vector ALUs.
//
// MFMA fragment conventions (v_mfma_f32_16x16x32_bf16 / _16x16x16bf16_1k, wave64):
//   A (16 x K): lane l holds row l%16 and K-slots [KPL*(l/16), KPL*(l/16)+KPL)
//   B (K x 16): lane l holds column l%16 and the same K-slots
//   D (16 x 16 fp32): lane l holds column l%16, rows 4*(l/16) + r, r = 0..3
// A contraction only needs A and B to enumerate K in the same order, so the K order below is
// chosen to match the D layout of the producing product ("slot kappa"): for a 32-wide K step m
// over keys, slot r' of lane group g is key 32m + 16*(r'/4) + 4g + r'%4.  With that order the
// squared-score tile (computed transposed, keys as rows) is directly the A operand of P.V, and
// the fp32 state tiles are directly the B operand of the readout.
#include "device.h"
#include "kata.h"

namespace kata {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int P = 16, DV = 64, C = 64, F = P * P;
constexpr int kThreads = 256;
constexpr int kStateFloats = F * (DV + 1);     // 16640: S (4 waves x 16 tiles x 256) + Z (256)
constexpr int QROW = 24;                       // bf16 per row of the Q / K tiles (16 + pad)
constexpr int KTROW = 68;                      // fp32 per row of the K^T tile (64 + pad)
constexpr int VTROW = 72;                      // bf16 per row of the V^T tile (64 + pad)

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- chunk tiles in LDS ------------------------------------------------------------------
struct __align__(16) Tiles {
  __bf16 Qs[C][QROW];     // q rows (bf16), row-major
  __bf16 Ks[C][QROW];     // k rows (bf16), row-major
  float KT[P][KTROW];     // k transposed, fp32 (exact copies of the bf16 inputs)
  __bf16 VT[DV][VTROW];   // v transposed, bf16
};

// One thread's share of a chunk's global loads, held in registers while the previous chunk
// is computed.  Threads 0..127 carry half a q row, 128..255 half a k row; every thread
// carries 16 bytes of two consecutive v rows.
struct Stage {
  uint4 qk;
  uint4 v0, v1;
};

__device__ __forceinline__ uint4 ld16(const __bf16* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ void stage_load(Stage& st, const DevProblem& pr, const __bf16* q,
                                           const __bf16* k, const __bf16* v, int b, int h,
                                           int tok0, bool with_q, int tid) {
  const int half = tid & 1;
  if (tid < 128) {
    if (with_q) st.qk = ld16(q + row_off(pr.sq, b, tok0 + (tid >> 1), h) + 8 * half);
  } else {
    st.qk = ld16(k + row_off(pr.sk, b, tok0 + ((tid - 128) >> 1), h) + 8 * half);
  }
  const int a = tid >> 3, c8 = tid & 7;
  st.v0 = ld16(v + row_off(pr.sv, b, tok0 + 2 * a, h) + 8 * c8);
  st.v1 = ld16(v + row_off(pr.sv, b, tok0 + 2 * a + 1, h) + 8 * c8);
}

__device__ __forceinline__ void stage_store(const Stage& st, Tiles& tl, bool with_q, int tid) {
  const int half = tid & 1;
  if (tid < 128) {
    if (with_q) *reinterpret_cast<uint4*>(&tl.Qs[tid >> 1][8 * half]) = st.qk;
  } else {
    const int s = (tid - 128) >> 1;
    *reinterpret_cast<uint4*>(&tl.Ks[s][8 * half]) = st.qk;
    const uint32_t w[4] = {st.qk.x, st.qk.y, st.qk.z, st.qk.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tl.KT[8 * half + 2 * e][s] = bf_lo(w[e]);
      tl.KT[8 * half + 2 * e + 1][s] = bf_hi(w[e]);
    }
  }
  const int a = tid >> 3, c8 = tid & 7;
  const uint32_t w0[4] = {st.v0.x, st.v0.y, st.v0.z, st.v0.w};
  const uint32_t w1[4] = {st.v1.x, st.v1.y, st.v1.z, st.v1.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // column d = 8*c8 + 2e (low halves) and d + 1 (high halves); rows 2a, 2a+1 as one dword
    *reinterpret_cast<uint32_t*>(&tl.VT[8 * c8 + 2 * e][2 * a]) = (w0[e] & 0xffffu) | (w1[e] << 16);
    *reinterpret_cast<uint32_t*>(&tl.VT[8 * c8 + 2 * e + 1][2 * a]) = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
  }
}

// B operand of a 32-key step m for value columns [16 nt, 16 nt + 16), slot order kappa.
__device__ __forceinline__ bf16x8 v_frag(const Tiles& tl, int m, int nt, int lane) {
  const int d = 16 * nt + (lane & 15), g = lane >> 4;
  const uint2 lo = *reinterpret_cast<const uint2*>(&tl.VT[d][32 * m + 4 * g]);
  const uint2 hi = *reinterpret_cast<const uint2*>(&tl.VT[d][32 * m + 16 + 4 * g]);
  uint4 u = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, u);
}

// A operand of the state update for feature rows f = 16 i + (lane%16), i fixed, 32-key step
// m: phi_f(k_s) = k_s[i] k_s[j], slot order kappa.
__device__ __forceinline__ bf16x8 phik_frag(const Tiles& tl, int i, int m, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const float4 ia = *reinterpret_cast<const float4*>(&tl.KT[i][32 * m + 4 * g]);
  const float4 ib = *reinterpret_cast<const float4*>(&tl.KT[i][32 * m + 16 + 4 * g]);
  const float4 ja = *reinterpret_cast<const float4*>(&tl.KT[j][32 * m + 4 * g]);
  const float4 jb = *reinterpret_cast<const float4*>(&tl.KT[j][32 * m + 16 + 4 * g]);
  bf16x8 f;
  f[0] = (__bf16)(ia.x * ja.x); f[1] = (__bf16)(ia.y * ja.y);
  f[2] = (__bf16)(ia.z * ja.z); f[3] = (__bf16)(ia.w * ja.w);
  f[4] = (__bf16)(ib.x * jb.x); f[5] = (__bf16)(ib.y * jb.y);
  f[6] = (__bf16)(ib.z * jb.z); f[7] = (__bf16)(ib.w * jb.w);
  return f;
}

// k_s[i] for i = lane%16 over the slots of 32-key step m (A and B operand of Z = K^T K).
__device__ __forceinline__ bf16x8 kcol_frag(const Tiles& tl, int m, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const float4 a = *reinterpret_cast<const float4*>(&tl.KT[i][32 * m + 4 * g]);
  const float4 c = *reinterpret_cast<const float4*>(&tl.KT[i][32 * m + 16 + 4 * g]);
  bf16x8 f;
  f[0] = (__bf16)a.x; f[1] = (__bf16)a.y; f[2] = (__bf16)a.z; f[3] = (__bf16)a.w;
  f[4] = (__bf16)c.x; f[5] = (__bf16)c.y; f[6] = (__bf16)c.z; f[7] = (__bf16)c.w;
  return f;
}

// 16 x 16 x 16 operand: row (lane%16) of a row-major [.][QROW] tile, columns 4g..4g+3.
__device__ __forceinline__ s16x4 row4_frag(const __bf16 (*X)[QROW], int row0, int lane) {
  const uint2 u = *reinterpret_cast<const uint2*>(&X[row0 + (lane & 15)][4 * (lane >> 4)]);
  return __builtin_bit_cast(s16x4, u);
}

// Squared, causally masked score tile -> bf16 P slots and their fp32 row-sum share.
// sc holds S^T[s][t] for keys s = s0 + 4g + r and query t = t0 + lane%16.
__device__ __forceinline__ void square_mask(const f32x4& sc, int s0, int t, int lane,
                                            __bf16 out[4], float& lsum) {
  const int g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = s0 + 4 * g + r;
    const float x = sc[r];
    const __bf16 pb = (s <= t) ? (__bf16)(x * x) : (__bf16)0.f;   // select, never multiply
    out[r] = pb;
    lsum += (float)pb;
  }
}

template <typename Tout>
__device__ __forceinline__ Tout cvt_out(float x) { return from_f32<Tout>(x); }

// ==========================================================================================
// Segment state: S_seg = sum over the segment's chunks of Phi(K_c)^T V_c and Z_seg = sum K^T K.
// Grid (n_seg, H, B).  Wave w owns feature rows [64 w, 64 w + 64) x all 64 value columns.
// ==========================================================================================
__global__ __launch_bounds__(kThreads, 2) void chunk_state_fast_kernel(
    DevProblem pr, int L, int n_seg, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, float* __restrict__ states) {
  __shared__ Tiles tl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int seg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);

  f32x4 S[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[mt][nt] = zero4();
  f32x4 Z = zero4();

  Stage st;
  stage_load(st, pr, nullptr, k, v, b, h, c0 * C, false, tid);
  stage_store(st, tl, false, tid);
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    if (c + 1 < nc) stage_load(st, pr, nullptr, k, v, b, h, (c0 + c + 1) * C, false, tid);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8 vb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) vb[nt] = v_frag(tl, m, nt, lane);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = phik_frag(tl, 4 * w + mt, m, lane);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) S[mt][nt] = mfma32(a, vb[nt], S[mt][nt]);
      }
      if (w == 0) {
        const bf16x8 kf = kcol_frag(tl, m, lane);
        Z = mfma32(kf, kf, Z);
      }
    }
    __syncthreads();
    if (c + 1 < nc) stage_store(st, tl, false, tid);
    __syncthreads();
  }
  float* out = states + ((long long)(b * pr.H + h) * n_seg + seg) * kStateFloats;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      *reinterpret_cast<f32x4*>(out + ((w * 16 + mt * 4 + nt) * 64 + lane) * 4) = S[mt][nt];
  if (w == 0) *reinterpret_cast<f32x4*>(out + F * DV + lane * 4) = Z;
}

// ==========================================================================================
// Segment walk: start from the segment's exclusive prefix (S_{<c}, Z_{<c}); for every chunk,
// outputs = (readout of the prefix + causal intra-chunk tile) / (eps + denominators), then
// the chunk's own state is added.  Grid (n_seg, H, B).
//   Wave w: owns state rows [64 w, 64 w + 64) (as in the state kernel), computes the readout
//   share of those rows for all 64 tokens, and finishes tokens [16 w, 16 w + 16): their intra
//   tile, the other waves' readout shares (through LDS), the denominator and the store.
// ==========================================================================================
struct __align__(16) WalkLds {
  Tiles tl;
  f32x4 red[4][3][4][64];        // readout shares for other waves' tokens
  float den[C];
};

template <typename Tout>
__global__ __launch_bounds__(kThreads, 2) void chunk_output_fast_kernel(
    DevProblem pr, int L, int n_seg, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den_out,
    const float* __restrict__ states) {
  __shared__ WalkLds sm;
  Tiles& tl = sm.tl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int seg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);

  // prefix state of this segment
  const float* pre = states + ((long long)(b * pr.H + h) * n_seg + seg) * kStateFloats;
  f32x4 S[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      S[mt][nt] = *reinterpret_cast<const f32x4*>(pre + ((w * 16 + mt * 4 + nt) * 64 + lane) * 4);
  // every wave keeps its own copy of Z_{<c} (4 registers); lane holds Z[4g + r][lane % 16]
  f32x4 Z = *reinterpret_cast<const f32x4*>(pre + F * DV + lane * 4);

  Stage st;
  stage_load(st, pr, q, k, v, b, h, c0 * C, true, tid);
  stage_store(st, tl, true, tid);
  __syncthreads();

  for (int c = 0; c < nc; ++c) {
    const int tok0 = (c0 + c) * C;
    if (c + 1 < nc) stage_load(st, pr, q, k, v, b, h, tok0 + C, true, tid);

    // ---- intra-chunk tile of this wave's tokens t in [16w, 16w+16) ----
    float lsum = 0.f;
    f32x4 Oown[4] = {zero4(), zero4(), zero4(), zero4()};
    {
      const s16x4 qf = row4_frag(tl.Qs, 16 * w, lane);
      const int t = 16 * w + l16;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (2 * m > w) break;                        // key tiles entirely in the future
        __bf16 pa[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int ms = 2 * m + half;
          if (ms <= w) {
            const f32x4 sc = mfma16(row4_frag(tl.Ks, 16 * ms, lane), qf, zero4());
            square_mask(sc, 16 * ms, t, lane, &pa[4 * half], lsum);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) pa[4 * half + r] = (__bf16)0.f;
          }
        }
        bf16x8 a;
#pragma unroll
        for (int r = 0; r < 8; ++r) a[r] = pa[r];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) Oown[nt] = mfma32(a, v_frag(tl, m, nt, lane), Oown[nt]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- inter-chunk denominator q^T Z_{<c} q for this wave's tokens ----
    // Y = Z q_t on MFMA with Z split into bf16 hi + lo (fp32-accurate; q is exact in bf16):
    // Z's accumulator layout (lane: column lane%16, rows 4g + r) is, Z being symmetric, the
    // A layout of a 16 x 16 x 16 product; q_t[4g..4g+3] is the same B operand as the scores.
    float zq = 0.f;
    {
      const s16x4 qf = row4_frag(tl.Qs, 16 * w, lane);
      s16x4 zhi, zlo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const __bf16 hi = (__bf16)Z[r];
        zhi[r] = __builtin_bit_cast(short, hi);
        zlo[r] = __builtin_bit_cast(short, (__bf16)(Z[r] - (float)hi));
      }
      f32x4 y = mfma16(zhi, qf, zero4());
      y = mfma16(zlo, qf, y);                   // y[r] = (Z q_t)[4g + r], t = 16w + lane%16
      const uint2 qq = __builtin_bit_cast(uint2, qf);
      zq = fmaf(bf_lo(qq.x), y[0], zq);
      zq = fmaf(bf_hi(qq.x), y[1], zq);
      zq = fmaf(bf_lo(qq.y), y[2], zq);
      zq = fmaf(bf_hi(qq.y), y[3], zq);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- readout of the prefix with rows [64w, 64w+64) of the state, one token tile at a
    // time; shares of other waves' tokens go to LDS, this wave's own share is kept.
    // (tt is a compile-time index after unrolling and w is uniform per wave, so no register
    // array is ever indexed at run time.)
    {
      bf16x8 sb[2][4];   // S as B operand: K step m' covers state tiles 2m', 2m'+1
#pragma unroll
      for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sb[mp][nt][r] = (__bf16)S[2 * mp][nt][r];
            sb[mp][nt][4 + r] = (__bf16)S[2 * mp + 1][nt][r];
          }
        }
#pragma unroll 1
      for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + l16;
        const uint2 qi = *reinterpret_cast<const uint2*>(&tl.Qs[t][4 * w]);   // q_t[4w..4w+3]
        const uint2 qj = *reinterpret_cast<const uint2*>(&tl.Qs[t][4 * g]);   // q_t[4g..4g+3]
        const float qiv[4] = {bf_lo(qi.x), bf_hi(qi.x), bf_lo(qi.y), bf_hi(qi.y)};
        const float qjv[4] = {bf_lo(qj.x), bf_hi(qj.x), bf_lo(qj.y), bf_hi(qj.y)};
        f32x4 O[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int mp = 0; mp < 2; ++mp) {
          // slot r' -> feature (i, j) = (4w + 2mp + r'/4, 4g + r'%4)
          bf16x8 a;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            a[r] = (__bf16)(qiv[2 * mp] * qjv[r]);
            a[4 + r] = (__bf16)(qiv[2 * mp + 1] * qjv[r]);
          }
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) O[nt] = mfma32(a, sb[mp][nt], O[nt]);
        }
        if (tt == w) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) Oown[nt] += O[nt];
        } else {
          const int slot = w < tt ? w : w - 1;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) sm.red[tt][slot][nt][lane] = O[nt];
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- state update with this chunk: S += Phi(K)^T V, Z += K^T K ----
#pragma unroll 1
    for (int m = 0; m < 2; ++m) {
      bf16x8 vb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) vb[nt] = v_frag(tl, m, nt, lane);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = phik_frag(tl, 4 * w + mt, m, lane);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) S[mt][nt] = mfma32(a, vb[nt], S[mt][nt]);
      }
      const bf16x8 kf = kcol_frag(tl, m, lane);
      Z = mfma32(kf, kf, Z);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- hand the other waves their readout shares; finish the denominators ----
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    zq += __shfl_xor(zq, 16);
    zq += __shfl_xor(zq, 32);
    if (g == 0) sm.den[16 * w + l16] = pr.eps + (zq + lsum);
    __syncthreads();

    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      acc[nt] = Oown[nt];
#pragma unroll
      for (int s2 = 0; s2 < 3; ++s2) acc[nt] += sm.red[w][s2][nt][lane];
    }
    // lane holds tokens 16w + 4g + r, value column 16 nt + l16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl_ = 16 * w + 4 * g + r;
      const float D = sm.den[tl_];
      const float inv = 1.f / D;
      Tout* op = o + row_off(pr.so, b, tok0 + tl_, h);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) op[16 * nt + l16] = cvt_out<Tout>(acc[nt][r] * inv);
    }
    if (den_out && lane < 16)
      den_out[((long long)b * pr.T + tok0 + 16 * w + lane) * pr.H + h] = sm.den[16 * w + lane];

    if (c + 1 < nc) stage_store(st, tl, true, tid);
    __syncthreads();
  }
}

// ==========================================================================================
// Flash-style quadratic forward: 64 queries per workgroup (16 per wave), key blocks of 64
// staged in LDS; scores, square + mask, P.V and the row sum, no running maximum (the scores
// are squares, so nothing needs rescaling).  Grid (ceil(T/64), H, B), heaviest blocks first.
// ==========================================================================================
struct __align__(16) QuadLds {
  __bf16 Ks[C][QROW];
  __bf16 VT[DV][VTROW];
  float den[C];
};

__device__ __forceinline__ void quad_stage_load(uint4& kq, uint4& v0, uint4& v1,
                                                const DevProblem& pr, const __bf16* k,
                                                const __bf16* v, int b, int h, int s0, int tid) {
  const uint4 z = {0u, 0u, 0u, 0u};
  if (tid < 128) {
    const int s = s0 + (tid >> 1);
    kq = s < pr.T ? ld16(k + row_off(pr.sk, b, s, h) + 8 * (tid & 1)) : z;
  }
  const int a = tid >> 3, c8 = tid & 7;
  const int s = s0 + 2 * a;
  v0 = s < pr.T ? ld16(v + row_off(pr.sv, b, s, h) + 8 * c8) : z;
  v1 = s + 1 < pr.T ? ld16(v + row_off(pr.sv, b, s + 1, h) + 8 * c8) : z;
}

__device__ __forceinline__ void quad_stage_store(const uint4& kq, const uint4& v0,
                                                 const uint4& v1, QuadLds& sm, int tid) {
  if (tid < 128) *reinterpret_cast<uint4*>(&sm.Ks[tid >> 1][8 * (tid & 1)]) = kq;
  const int a = tid >> 3, c8 = tid & 7;
  const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};
  const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    *reinterpret_cast<uint32_t*>(&sm.VT[8 * c8 + 2 * e][2 * a]) = (w0[e] & 0xffffu) | (w1[e] << 16);
    *reinterpret_cast<uint32_t*>(&sm.VT[8 * c8 + 2 * e + 1][2 * a]) = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
  }
}

template <typename Tout>
__global__ __launch_bounds__(kThreads, 2) void quadratic_fast_kernel(
    DevProblem pr, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den_out) {
  __shared__ QuadLds sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int qb = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = qb * C;
  const int t = t0 + 16 * w + l16;             // this lane's query (fragment column)

  // query operand of the score tile: q_t[4g..4g+3]
  s16x4 qf = {0, 0, 0, 0};
  if (t < pr.T)
    qf = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2*>(q + row_off(pr.sq, b, t, h) + 4 * g));

  f32x4 O[4] = {zero4(), zero4(), zero4(), zero4()};
  float lsum = 0.f;
  uint4 kq = {0u, 0u, 0u, 0u}, v0, v1;
  quad_stage_load(kq, v0, v1, pr, k, v, b, h, 0, tid);
  quad_stage_store(kq, v0, v1, sm, tid);
  __syncthreads();
  for (int kb = 0; kb <= qb; ++kb) {
    if (kb < qb) quad_stage_load(kq, v0, v1, pr, k, v, b, h, (kb + 1) * C, tid);
    const int s_base = kb * C;
    const bool diag = (kb == qb);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (diag && 2 * m > w) break;
      __bf16 pa[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ms = 2 * m + half;
        if (!diag || ms <= w) {
          const f32x4 sc = mfma16(row4_frag(sm.Ks, 16 * ms, lane), qf, zero4());
          square_mask(sc, s_base + 16 * ms, t, lane, &pa[4 * half], lsum);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) pa[4 * half + r] = (__bf16)0.f;
        }
      }
      bf16x8 a;
#pragma unroll
      for (int r = 0; r < 8; ++r) a[r] = pa[r];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int d = 16 * nt + l16;
        const uint2 lo = *reinterpret_cast<const uint2*>(&sm.VT[d][32 * m + 4 * g]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&sm.VT[d][32 * m + 16 + 4 * g]);
        const uint4 u = {lo.x, lo.y, hi.x, hi.y};
        O[nt] = mfma32(a, __builtin_bit_cast(bf16x8, u), O[nt]);
      }
    }
    __syncthreads();
    if (kb < qb) quad_stage_store(kq, v0, v1, sm, tid);
    __syncthreads();
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (g == 0) sm.den[16 * w + l16] = pr.eps + lsum;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tr = 16 * w + 4 * g + r;
    if (t0 + tr >= pr.T) continue;
    const float inv = 1.f / sm.den[tr];
    Tout* op = o + row_off(pr.so, b, t0 + tr, h);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) op[16 * nt + l16] = cvt_out<Tout>(O[nt][r] * inv);
  }
  if (den_out && lane < 16 && t0 + 16 * w + lane < pr.T)
    den_out[((long long)b * pr.T + t0 + 16 * w + lane) * pr.H + h] = sm.den[16 * w + lane];
}

}  // namespace

bool quadratic_fast_supported(const kata_problem* pr) {
  return pr->in_dtype == KATA_BF16 && pr->p == P && pr->dv == DV;
}

bool chunk_fast_available() { return true; }

hipError_t launch_quadratic_fast(const DevProblem& pr, bool out_bf16, const void* q,
                                 const void* k, const void* v, void* o, float* den,
                                 hipStream_t st) {
  dim3 grid((pr.T + C - 1) / C, pr.H, pr.B);
  if (out_bf16)
    quadratic_fast_kernel<__bf16><<<grid, kThreads, 0, st>>>(
        pr, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, den);
  else
    quadratic_fast_kernel<float><<<grid, kThreads, 0, st>>>(
        pr, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (float*)o, den);
  return hipGetLastError();
}

hipError_t launch_chunk_state_fast(const DevProblem& pr, int L, int n_seg, const void* k,
                                   const void* v, float* states, hipStream_t st) {
  if (pr.p != P || pr.dv != DV || pr.C != C) return hipErrorInvalidValue;
  dim3 grid(n_seg, pr.H, pr.B);
  chunk_state_fast_kernel<<<grid, kThreads, 0, st>>>(pr, L, n_seg, (const __bf16*)k,
                                                     (const __bf16*)v, states);
  return hipGetLastError();
}

hipError_t launch_chunk_output_fast(const DevProblem& pr, bool out_bf16, int L, int n_seg,
                                    const void* q, const void* k, const void* v, void* o,
                                    float* den, const float* states, hipStream_t st) {
  if (pr.p != P || pr.dv != DV || pr.C != C) return hipErrorInvalidValue;
  dim3 grid(n_seg, pr.H, pr.B);
  if (out_bf16)
    chunk_output_fast_kernel<__bf16><<<grid, kThreads, 0, st>>>(
        pr, L, n_seg, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, den,
        states);
  else
    chunk_output_fast_kernel<float><<<grid, kThreads, 0, st>>>(
        pr, L, n_seg, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (float*)o, den,
        states);
  return hipGetLastError();
}

}  // namespace kata

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
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int P = 16, DV = 64, C = 64, F = P * P;
constexpr int kThreads = 256;
constexpr int kStateFloats = F * (DV + 1);     // 16640: S (4 waves x 16 tiles x 256) + Z (256)
// LDS row strides, chosen so that every access pattern below is free of bank conflicts
// (32 banks of 4 bytes; 4-, 8- and 16-byte accesses served 32, 16 and 8 lanes at a time):
constexpr int QROW = 20;                       // bf16 per q / k row: 40 B, 8-byte aligned
constexpr int KTROW = 68;                      // fp32 per row of the K^T tile
constexpr int VROW = 80;                       // bf16 per v row: 160 B, 16-byte aligned

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
  __bf16 V[C][VROW];      // v rows (bf16), row-major
};

// One thread's share of a chunk's global loads, held in registers while the previous chunk
// is computed.  Waves 0-1 carry half a q row each (token = lane, half = wave), waves 2-3 half
// a k row; every thread carries 16 bytes of two consecutive v rows.
struct Stage {
  uint4 qk;
  uint4 v0, v1;
};

__device__ __forceinline__ uint4 ld16(const __bf16* p) { return *reinterpret_cast<const uint4*>(p); }

// Per-thread global addresses of the staged pieces; advanced by one chunk with `next`.
struct StagePtrs {
  const __bf16* qk;     // q (waves 0-1) or k (waves 2-3) piece, or nullptr
  const __bf16* v0;     // v row 2a, 16 bytes at column 8 c8
  long long qk_step, v_step;
  __device__ __forceinline__ void next() {
    if (qk) qk += qk_step;
    v0 += v_step;
  }
};

__device__ __forceinline__ StagePtrs stage_ptrs(const DevProblem& pr, const __bf16* q,
                                                const __bf16* k, const __bf16* v, int b, int h,
                                                int tok0, bool with_q, int tid, int dir = 1) {
  StagePtrs sp;
  const int w = tid >> 6, lane = tid & 63;
  if (w < 2)
    sp.qk = with_q ? q + row_off(pr.sq, b, tok0 + lane, h) + 8 * w : nullptr;
  else
    sp.qk = k + row_off(pr.sk, b, tok0 + lane, h) + 8 * (w - 2);
  sp.qk_step = (long long)dir * C * (w < 2 ? pr.sq[1] : pr.sk[1]);
  const int a = tid >> 3, c8 = tid & 7;
  sp.v0 = v + row_off(pr.sv, b, tok0 + 2 * a, h) + 8 * c8;
  sp.v_step = (long long)dir * C * pr.sv[1];
  return sp;
}

__device__ __forceinline__ void stage_load(Stage& st, const StagePtrs& sp, long long sv_t) {
  if (sp.qk) st.qk = ld16(sp.qk);
  st.v0 = ld16(sp.v0);
  st.v1 = ld16(sp.v0 + sv_t);
}

__device__ __forceinline__ void stage_store(const Stage& st, Tiles& tl, bool with_q, int tid) {
  const int w = tid >> 6, lane = tid & 63;
  if (w < 2) {
    if (with_q) {
      *reinterpret_cast<uint2*>(&tl.Qs[lane][8 * w]) = uint2{st.qk.x, st.qk.y};
      *reinterpret_cast<uint2*>(&tl.Qs[lane][8 * w + 4]) = uint2{st.qk.z, st.qk.w};
    }
  } else {
    const int half = w - 2;
    *reinterpret_cast<uint2*>(&tl.Ks[lane][8 * half]) = uint2{st.qk.x, st.qk.y};
    *reinterpret_cast<uint2*>(&tl.Ks[lane][8 * half + 4]) = uint2{st.qk.z, st.qk.w};
    const uint32_t wd[4] = {st.qk.x, st.qk.y, st.qk.z, st.qk.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tl.KT[8 * half + 2 * e][lane] = bf_lo(wd[e]);
      tl.KT[8 * half + 2 * e + 1][lane] = bf_hi(wd[e]);
    }
  }
  const int a = tid >> 3, c8 = tid & 7;
  *reinterpret_cast<uint4*>(&tl.V[2 * a][8 * c8]) = st.v0;
  *reinterpret_cast<uint4*>(&tl.V[2 * a + 1][8 * c8]) = st.v1;
}

// B operand of a 32-key step m for value columns [16 nt, 16 nt + 16), slot order kappa, read
// from the row-major V tile with two LDS transpose loads.  Within a 16-lane block, lane i's
// slot r of ds_read_b64_tr_b16 is element (i % 4) of the 8 bytes addressed by block lane
// 4r + i/4; block lane j therefore points at V[key(g, j/4)][16 nt + 4 (j % 4)], which hands
// lane i the value V[key(g, r)][16 nt + i].
__device__ __forceinline__ bf16x8 v_frag(const __bf16 (*V)[VROW], int m, int nt, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int row = 32 * m + 4 * g + (j >> 2), col = 16 * nt + 4 * (j & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&V[row][col]));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&V[row + 16][col]));
  const uint2 ul = __builtin_bit_cast(uint2, lo), uh = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, uint4{ul.x, ul.y, uh.x, uh.y});
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
template <bool kMask>
__device__ __forceinline__ void square_mask(const f32x4& sc, int s0, int t, int lane,
                                            __bf16 out[4], float& lsum) {
  const int g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float x = sc[r];
    __bf16 pb = (__bf16)(x * x);
    if (kMask) pb = (s0 + 4 * g + r <= t) ? pb : (__bf16)0.f;   // select, never multiply
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
__global__ __launch_bounds__(kThreads, 3) void chunk_state_fast_kernel(
    DevProblem pr, int L, int n_seg, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, float* __restrict__ states) {
  __shared__ Tiles tl[2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int seg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);
  const long long sv_t = pr.sv[1];

  f32x4 S[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[mt][nt] = zero4();
  f32x4 Z = zero4();

  // The sum is order-free, so the segment is read last chunk first: the walk that follows
  // starts at the segment's first chunks, which are then the most recently read.  Two chunks
  // are in flight in registers (loaded two iterations before they are staged into LDS); the
  // loop is unrolled by two so the register ring is indexed at compile time only.
  StagePtrs sp = stage_ptrs(pr, nullptr, k, v, b, h, (c0 + nc - 1) * C, false, tid, -1);
  Stage sa, sb;
  stage_load(sa, sp, sv_t);
  stage_store(sa, tl[0], false, tid);
  if (nc > 1) { sp.next(); stage_load(sa, sp, sv_t); }
  if (nc > 2) { sp.next(); stage_load(sb, sp, sv_t); }
  __syncthreads();
  auto step = [&](int c, Stage& next, Stage& after) {
    const Tiles& cur = tl[c & 1];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8 vb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) vb[nt] = v_frag(cur.V, m, nt, lane);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = phik_frag(cur, 4 * w + mt, m, lane);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) S[mt][nt] = mfma32(a, vb[nt], S[mt][nt]);
      }
      if (w == 0) {
        const bf16x8 kf = kcol_frag(cur, m, lane);
        Z = mfma32(kf, kf, Z);
      }
    }
    // the other buffer was last read in the previous iteration, before its barrier
    if (c + 1 < nc) stage_store(next, tl[(c + 1) & 1], false, tid);
    if (c + 3 < nc) { sp.next(); stage_load(next, sp, sv_t); }   // chunk c + 3
    __syncthreads();
    (void)after;
  };
  for (int c = 0; c < nc; c += 2) {
    step(c, sa, sb);                 // chunk c+1 is in sa, chunk c+2 in sb
    if (c + 1 < nc) step(c + 1, sb, sa);
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
//   Wave w owns state rows [64 w, 64 w + 64) (fp32, in registers, as in the state kernel) and
//   the chunk's tokens [16 w, 16 w + 16).  Once per chunk every wave publishes its state rows
//   in LDS as bf16 B operands; each wave then reads out its own tokens over all 256 rows, so
//   no partial outputs cross waves.
// ==========================================================================================
struct __align__(16) WalkLds {
  Tiles tl;
  uint4 Sb[8][4][64];            // S_{<c} as B operands: [32-row K step][value tile][lane]
  float den[C];                  // D_t of the chunk's tokens
  float inv[C];                  // 1 / D_t
};

template <typename Tout>
__global__ __launch_bounds__(kThreads, 3) void chunk_output_fast_kernel(
    DevProblem pr, int L, int n_seg, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den_out,
    const float* __restrict__ states) {
  __shared__ WalkLds sm;
  Tiles& tl = sm.tl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int seg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);
  const long long sv_t = pr.sv[1];

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

  // publish this wave's state rows as bf16 B operands: K step 2w + mp covers state tiles
  // 2mp, 2mp+1 of this wave (slot r' -> row 16 (4w + 2mp + r'/4) + 4g + r'%4)
  auto publish = [&]() {
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        bf16x8 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = (__bf16)S[2 * mp][nt][r];
          x[4 + r] = (__bf16)S[2 * mp + 1][nt][r];
        }
        sm.Sb[2 * w + mp][nt][lane] = __builtin_bit_cast(uint4, x);
      }
  };

  StagePtrs sp = stage_ptrs(pr, q, k, v, b, h, c0 * C, true, tid);
  Stage st;
  stage_load(st, sp, sv_t);
  stage_store(st, tl, true, tid);
  publish();
  __syncthreads();

  // output row pointer of this lane's first token (16w + 4g) in the first chunk
  Tout* orow = o + row_off(pr.so, b, c0 * C + 16 * w + 4 * g, h) + l16;
  const long long so_t = pr.so[1];

  for (int c = 0; c < nc; ++c) {
    const int tok0 = (c0 + c) * C;
    if (c + 1 < nc) {
      sp.next();
      stage_load(st, sp, sv_t);
    }
    const int t = 16 * w + l16;                  // this lane's token (fragment column / row)

    // ---- intra-chunk tile of this wave's tokens ----
    float lsum = 0.f;
    f32x4 O[4] = {zero4(), zero4(), zero4(), zero4()};
    const s16x4 qf = row4_frag(tl.Qs, 16 * w, lane);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (2 * m > w) break;                        // key tiles entirely in the future
      __bf16 pa[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ms = 2 * m + half;
        if (ms < w) {
          const f32x4 sc = mfma16(row4_frag(tl.Ks, 16 * ms, lane), qf, zero4());
          square_mask<false>(sc, 16 * ms, t, lane, &pa[4 * half], lsum);
        } else if (ms == w) {
          const f32x4 sc = mfma16(row4_frag(tl.Ks, 16 * ms, lane), qf, zero4());
          square_mask<true>(sc, 16 * ms, t, lane, &pa[4 * half], lsum);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) pa[4 * half + r] = (__bf16)0.f;
        }
      }
      bf16x8 a;
#pragma unroll
      for (int r = 0; r < 8; ++r) a[r] = pa[r];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) O[nt] = mfma32(a, v_frag(tl.V, m, nt, lane), O[nt]);
    }

    // ---- inter-chunk denominator q^T Z_{<c} q ----
    // Y = Z q_t on MFMA with Z split into bf16 hi + lo (fp32-accurate; q is exact in bf16):
    // Z's accumulator layout (lane: column lane%16, rows 4g + r) is, Z being symmetric, the
    // A layout of a 16 x 16 x 16 product; q_t[4g..4g+3] is the same B operand as the scores.
    float zq = 0.f;
    {
      s16x4 zhi, zlo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const __bf16 hi = (__bf16)Z[r];
        zhi[r] = __builtin_bit_cast(short, hi);
        zlo[r] = __builtin_bit_cast(short, (__bf16)(Z[r] - (float)hi));
      }
      f32x4 y = mfma16(zhi, qf, zero4());
      y = mfma16(zlo, qf, y);                   // y[r] = (Z q_t)[4g + r]
      const uint2 qq = __builtin_bit_cast(uint2, qf);
      zq = fmaf(bf_lo(qq.x), y[0], zq);
      zq = fmaf(bf_hi(qq.x), y[1], zq);
      zq = fmaf(bf_lo(qq.y), y[2], zq);
      zq = fmaf(bf_hi(qq.y), y[3], zq);
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    zq += __shfl_xor(zq, 16);
    zq += __shfl_xor(zq, 32);
    if (g == 0) {
      const float D = pr.eps + (zq + lsum);
      sm.den[t] = D;
      sm.inv[t] = 1.f / D;
    }

    // ---- readout phi(q_t)^T S_{<c} over all 256 state rows (8 K steps of 32) ----
    {
      const uint4 q0 = *reinterpret_cast<const uint4*>(&tl.Qs[t][0]);
      const uint4 q1 = *reinterpret_cast<const uint4*>(&tl.Qs[t][8]);
      const float qv[16] = {bf_lo(q0.x), bf_hi(q0.x), bf_lo(q0.y), bf_hi(q0.y),
                            bf_lo(q0.z), bf_hi(q0.z), bf_lo(q0.w), bf_hi(q0.w),
                            bf_lo(q1.x), bf_hi(q1.x), bf_lo(q1.y), bf_hi(q1.y),
                            bf_lo(q1.z), bf_hi(q1.z), bf_lo(q1.w), bf_hi(q1.w)};
      const uint2 q4 = *reinterpret_cast<const uint2*>(&tl.Qs[t][4 * g]);
      const float qj[4] = {bf_lo(q4.x), bf_hi(q4.x), bf_lo(q4.y), bf_hi(q4.y)};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        // slot r' -> feature (i, j) = (2kk + r'/4, 4g + r'%4)
        bf16x8 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] = (__bf16)(qv[2 * kk] * qj[r]);
          a[4 + r] = (__bf16)(qv[2 * kk + 1] * qj[r]);
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          O[nt] = mfma32(a, __builtin_bit_cast(bf16x8, sm.Sb[kk][nt][lane]), O[nt]);
      }
    }

    // ---- gate and store this wave's tokens: lane holds tokens 16w + 4g + r, column 16nt + l16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float inv = sm.inv[16 * w + 4 * g + r];
      Tout* op = orow + r * so_t;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)   // streamed out: never re-read by this kernel
        __builtin_nontemporal_store(cvt_out<Tout>(O[nt][r] * inv), op + 16 * nt);
    }
    if (den_out && lane < 16)
      den_out[((long long)b * pr.T + tok0 + 16 * w + lane) * pr.H + h] = sm.den[16 * w + lane];
    orow += C * so_t;

    // ---- state update with this chunk: S += Phi(K)^T V, Z += K^T K ----
#pragma unroll 1
    for (int m = 0; m < 2; ++m) {
      bf16x8 vb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) vb[nt] = v_frag(tl.V, m, nt, lane);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = phik_frag(tl, 4 * w + mt, m, lane);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) S[mt][nt] = mfma32(a, vb[nt], S[mt][nt]);
      }
      const bf16x8 kf = kcol_frag(tl, m, lane);
      Z = mfma32(kf, kf, Z);
    }
    __syncthreads();                               // all reads of this chunk's tiles and Sb done
    if (c + 1 < nc) {
      stage_store(st, tl, true, tid);
      publish();
    }
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
  __bf16 V[C][VROW];
  float inv[C];
  float den[C];
};

template <typename Tout>
__global__ __launch_bounds__(kThreads, 2) void quadratic_fast_kernel(
    DevProblem pr, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, Tout* __restrict__ o, float* __restrict__ den_out) {
  __shared__ QuadLds sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int qb = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = qb * C;
  const int t = t0 + 16 * w + l16;             // this lane's query (fragment column)
  const uint4 z4 = {0u, 0u, 0u, 0u};

  // query operand of the score tile: q_t[4g..4g+3]
  s16x4 qf = {0, 0, 0, 0};
  if (t < pr.T)
    qf = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2*>(q + row_off(pr.sq, b, t, h) + 4 * g));

  // staging: waves 0-1 half a k row each (key = lane), every thread 16 B of two v rows
  const int a = tid >> 3, c8 = tid & 7;
  auto load = [&](int s0) {
    Stage x;
    x.qk = z4;
    if (w < 2) {
      const int s = s0 + lane;
      x.qk = s < pr.T ? ld16(k + row_off(pr.sk, b, s, h) + 8 * w) : z4;
    }
    const int s = s0 + 2 * a;
    x.v0 = s < pr.T ? ld16(v + row_off(pr.sv, b, s, h) + 8 * c8) : z4;
    x.v1 = s + 1 < pr.T ? ld16(v + row_off(pr.sv, b, s + 1, h) + 8 * c8) : z4;
    return x;
  };
  auto store = [&](const Stage& x) {
    if (w < 2) {
      *reinterpret_cast<uint2*>(&sm.Ks[lane][8 * w]) = uint2{x.qk.x, x.qk.y};
      *reinterpret_cast<uint2*>(&sm.Ks[lane][8 * w + 4]) = uint2{x.qk.z, x.qk.w};
    }
    *reinterpret_cast<uint4*>(&sm.V[2 * a][8 * c8]) = x.v0;
    *reinterpret_cast<uint4*>(&sm.V[2 * a + 1][8 * c8]) = x.v1;
  };

  f32x4 O[4] = {zero4(), zero4(), zero4(), zero4()};
  float lsum = 0.f;
  Stage x = load(0);
  store(x);
  __syncthreads();
  for (int kb = 0; kb <= qb; ++kb) {
    if (kb < qb) x = load((kb + 1) * C);
    const int s_base = kb * C;
    const bool diag = (kb == qb);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (diag && 2 * m > w) break;
      __bf16 pa[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ms = 2 * m + half;
        if (!diag || ms < w) {
          const f32x4 sc = mfma16(row4_frag(sm.Ks, 16 * ms, lane), qf, zero4());
          square_mask<false>(sc, s_base + 16 * ms, t, lane, &pa[4 * half], lsum);
        } else if (ms == w) {
          const f32x4 sc = mfma16(row4_frag(sm.Ks, 16 * ms, lane), qf, zero4());
          square_mask<true>(sc, s_base + 16 * ms, t, lane, &pa[4 * half], lsum);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) pa[4 * half + r] = (__bf16)0.f;
        }
      }
      bf16x8 af;
#pragma unroll
      for (int r = 0; r < 8; ++r) af[r] = pa[r];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) O[nt] = mfma32(af, v_frag(sm.V, m, nt, lane), O[nt]);
    }
    __syncthreads();
    if (kb < qb) store(x);
    __syncthreads();
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (g == 0) {
    const float D = pr.eps + lsum;
    sm.den[16 * w + l16] = D;
    sm.inv[16 * w + l16] = 1.f / D;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tr = 16 * w + 4 * g + r;
    if (t0 + tr >= pr.T) continue;
    const float inv = sm.inv[tr];
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

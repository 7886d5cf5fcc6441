// bf16 MFMA kernels for gfx950 at p = 32, d_v = 64, chunk C = 64: the chunk-state build and
// the segment walk of the chunked forward.  (The quadratic form is in quadratic.hip.)
//
// Same method and precision as the p = 16 kernels (gist.science "Technische Samenvatting"
// sections 2.1-2.3; ai.info AI summary, Main Findings): a_ts = (q_t . k_s)^2, bf16 MFMA
// products with fp32 accumulation, P rounded to bf16 with the row sum taken from the rounded
// values, fp32 running state, inter-chunk denominator q^T Z q in fp32 (Z split into bf16 hi +
// lo on MFMA).
//
// The state is always packed (the 528 unique pairs i <= j of the 32 x 32 feature, the ai.info
// state-size bullet's packed coordinates): 72 double groups = 36 tiles of 16 rows, 18 readout
// K steps.  That is 147 KB of fp32 per state, too much for four waves' registers, so a
// workgroup has eight waves (two per SIMD, one workgroup per CU):
//   state tiles  wave w owns tiles rank(w) + 8 s (5 tiles for ranks 0-3, 4 for ranks 4-7; the
//                waves with the most intra-chunk work own fewer),
//   tokens       wave w serves tokens [16 tg, 16 tg + 16) of a chunk, tg = w % 4, and the value
//                columns [32 ch, 32 ch + 32), ch = w / 4.  The two waves of a token group
//                split the readout's K steps instead of its columns (each forms phi(q) for
//                half the features, the VALU cost of the readout) and swap the partial sums
//                of each other's columns through LDS.
#include "device.h"
#include "kata.h"
#include "mfma_util.h"

namespace kata {
namespace {

constexpr int P = 32, DV = 64, C = 64;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kTiles = 36, kSteps = 18, kSlots = 5;
constexpr int kZOff = kTiles * 16 * DV;              // 36864
constexpr int kStateFloats = kZOff + 4 * 256;        // + Z as 2 x 2 tiles of 16 x 16
static_assert(kStateFloats == 36 * 16 * 64 + 4 * 256, "packed p = 32 state size (plan.h)");
constexpr int QROW = 40;                             // bf16 per q / k row: 80 B
constexpr int KTROW = 68;                            // fp32 per K^T row
constexpr int VROW = 80;                             // bf16 per v row: 160 B
constexpr int KTROWS = 2 * P + 1;                    // k, 2 k, zeros

struct __align__(16) Tiles32 {
  __bf16 Qs[C][QROW];
  __bf16 Ks[C][QROW];
  float KT[KTROWS][KTROW];
  __bf16 V[C][VROW];
};

struct __align__(16) StateTiles32 {                  // the state pass needs no q and no k rows
  float KT[KTROWS][KTROW];
  __bf16 V[C][VROW];
};

// waves in the order that receives 5, 5, 5, 5, 4, 4, 4, 4 tiles: token groups 0 and 1 first
__device__ __forceinline__ int wave_rank(int w) { return (w & 1) | ((w >> 2) << 1) | (((w >> 1) & 1) << 2); }
__device__ __forceinline__ bool owns(int w, int s) { return wave_rank(w) + 8 * s < kTiles; }
__device__ __forceinline__ int tile_of(int w, int s) { return wave_rank(w) + 8 * s; }

// One thread's share of a chunk's loads: threads 0-255 a quarter q row, 256-511 a quarter
// k row (row = (tid & 255) / 4, columns 8 (tid % 4) ..), every thread 16 B of one v row
// (row tid / 8, columns 8 (tid % 8) ..).
struct Stage32 {
  uint4 qk, v;
};

struct Ptrs32 {
  const __bf16* qk;
  const __bf16* v;
  long long qk_step, v_step;
  __device__ __forceinline__ void next() {
    if (qk) qk += qk_step;
    v += v_step;
  }
};

__device__ __forceinline__ Ptrs32 ptrs32(const DevProblem& pr, const __bf16* q, const __bf16* k,
                                         const __bf16* v, int b, int h, int tok0, bool with_q,
                                         int tid, int dir) {
  Ptrs32 p;
  const int lo = tid & 255, row = lo >> 2, qc = lo & 3;
  if (tid < 256) {
    p.qk = with_q ? q + row_off(pr.sq, b, tok0 + row, h) + 8 * qc : nullptr;
    p.qk_step = (long long)dir * C * pr.sq[1];
  } else {
    p.qk = k + row_off(pr.sk, b, tok0 + row, h) + 8 * qc;
    p.qk_step = (long long)dir * C * pr.sk[1];
  }
  p.v = v + row_off(pr.sv, b, tok0 + (tid >> 3), h) + 8 * (tid & 7);
  p.v_step = (long long)dir * C * pr.sv[1];
  return p;
}

__device__ __forceinline__ void load32(Stage32& s, const Ptrs32& p) {
  if (p.qk) s.qk = ld16(p.qk);
  s.v = ld16(p.v);
}

// k piece -> K^T rows (k, 2 k); q / k piece -> row-major rows (when the tile has them)
template <class TL>
__device__ __forceinline__ void store_kt(const Stage32& s, TL& tl, int tid) {
  const int lo = tid & 255, row = lo >> 2, qc = lo & 3;
  const uint32_t wd[4] = {s.qk.x, s.qk.y, s.qk.z, s.qk.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = bf_lo(wd[e]), c = bf_hi(wd[e]);
    tl.KT[8 * qc + 2 * e][row] = a;
    tl.KT[8 * qc + 2 * e + 1][row] = c;
    tl.KT[P + 8 * qc + 2 * e][row] = 2.f * a;           // exact
    tl.KT[P + 8 * qc + 2 * e + 1][row] = 2.f * c;
  }
}

__device__ __forceinline__ void store32(const Stage32& s, Tiles32& tl, bool with_q, int tid) {
  const int lo = tid & 255, row = lo >> 2, qc = lo & 3;
  if (tid < 256) {
    if (with_q) *reinterpret_cast<uint4*>(&tl.Qs[row][8 * qc]) = s.qk;
  } else {
    *reinterpret_cast<uint4*>(&tl.Ks[row][8 * qc]) = s.qk;
    store_kt(s, tl, tid);
  }
  *reinterpret_cast<uint4*>(&tl.V[tid >> 3][8 * (tid & 7)]) = s.v;
}

__device__ __forceinline__ void store_state32(const Stage32& s, StateTiles32& tl, int tid) {
  if (tid >= 256) store_kt(s, tl, tid);
  *reinterpret_cast<uint4*>(&tl.V[tid >> 3][8 * (tid & 7)]) = s.v;
}

template <class TL>
__device__ __forceinline__ void zero_row(TL& tl, int tid) {
  if (tid < KTROW) tl.KT[2 * P][tid] = 0.f;
}

// A operand of the packed update for this lane's tile row (irow selects k_i, 2 k_i or zeros),
// 32-key step m in slot order kappa.
template <class TL>
__device__ __forceinline__ bf16x8 phik(const TL& tl, int irow, int jrow, int m, int lane) {
  const int g = lane >> 4;
  const float4 ia = *reinterpret_cast<const float4*>(&tl.KT[irow][32 * m + 4 * g]);
  const float4 ib = *reinterpret_cast<const float4*>(&tl.KT[irow][32 * m + 16 + 4 * g]);
  const float4 ja = *reinterpret_cast<const float4*>(&tl.KT[jrow][32 * m + 4 * g]);
  const float4 jb = *reinterpret_cast<const float4*>(&tl.KT[jrow][32 * m + 16 + 4 * g]);
  bf16x8 f;
  f[0] = (__bf16)(ia.x * ja.x); f[1] = (__bf16)(ia.y * ja.y);
  f[2] = (__bf16)(ia.z * ja.z); f[3] = (__bf16)(ia.w * ja.w);
  f[4] = (__bf16)(ib.x * jb.x); f[5] = (__bf16)(ib.y * jb.y);
  f[6] = (__bf16)(ib.z * jb.z); f[7] = (__bf16)(ib.w * jb.w);
  return f;
}

// k_s[16 mi + lane%16] over the slots of 32-key step m (operand of Z = K^T K)
template <class TL>
__device__ __forceinline__ bf16x8 kcol(const TL& tl, int mi, int m, int lane) {
  const int i = 16 * mi + (lane & 15), g = lane >> 4;
  const float4 a = *reinterpret_cast<const float4*>(&tl.KT[i][32 * m + 4 * g]);
  const float4 c = *reinterpret_cast<const float4*>(&tl.KT[i][32 * m + 16 + 4 * g]);
  bf16x8 f;
  f[0] = (__bf16)a.x; f[1] = (__bf16)a.y; f[2] = (__bf16)a.z; f[3] = (__bf16)a.w;
  f[4] = (__bf16)c.x; f[5] = (__bf16)c.y; f[6] = (__bf16)c.z; f[7] = (__bf16)c.w;
  return f;
}

// Row sources of this lane's row of each owned tile.
struct Rows32 {
  int irow[kSlots], jrow[kSlots];
  __device__ void init(int w, int lane) {
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int t = owns(w, sl) ? tile_of(w, sl) : 0, row = lane & 15;
      int a, J;
      double_group(4 * (t >> 1) + (row >> 2), a, J);
      const int i = a + (t & 1), j = 4 * J + (row & 3);
      irow[sl] = i > j ? 2 * P : (i == j ? i : P + i);
      jrow[sl] = j;
    }
  }
};

// S[slot] += Phi(K)^T V over one staged chunk; Z += K^T K for the 16 x 16 tile
// (z >> 1, z & 1) when z >= 0 (waves 0-3 own one tile each).
template <class TL>
__device__ __forceinline__ void update32(const TL& tl, const Rows32& rw, f32x4 (&S)[kSlots][4],
                                         f32x4 (&Z)[2][2], int w, int lane, int z) {
  // both 32-key steps unrolled: the LDS addresses of the second become immediate offsets
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    bf16x8 vb[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) vb[nt] = v_frag(tl.V, m, nt, lane);
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      if (!owns(w, sl)) continue;
      const bf16x8 a = phik(tl, rw.irow[sl], rw.jrow[sl], m, lane);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[sl][nt] = mfma32(a, vb[nt], S[sl][nt]);
    }
    if (z >= 0) {                                  // wave-uniform
      const int mi = z >> 1, kj = z & 1;
      const bf16x8 a = kcol(tl, mi, m, lane), bb = kcol(tl, kj, m, lane);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          if (x == mi && y == kj) Z[x][y] = mfma32(a, bb, Z[x][y]);
    }
  }
}

// ==========================================================================================
// Segment state: S_seg = sum over the segment's chunks of Phi(K_c)^T V_c, Z_seg = sum K^T K.
// One workgroup per (segment, head, batch) (SegGrid); segments seg >= n_used get a zero state
// without reading their tokens.
// State layout (floats): tile t, value tile nt, lane -> ((t * 4 + nt) * 64 + lane) * 4, then
// Z tile (mi, kj) -> kZOff + ((mi * 2 + kj) * 64 + lane) * 4.
// ==========================================================================================
__global__ __launch_bounds__(kThreads, 1) void chunk_state32_kernel(
    DevProblem pr, SegGrid sg, int L, int n_seg, int n_used, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, float* __restrict__ states) {
  extern __shared__ __align__(16) unsigned char smem[];
  StateTiles32* tl = reinterpret_cast<StateTiles32*>(smem);    // two buffers
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const SegBlock blk = seg_block(sg, pr.H);
  if (!blk.live) return;                           // padding of the grid (whole workgroup)
  const int seg = blk.seg, h = blk.h, b = blk.b;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);
  float* out = states + ((long long)(b * pr.H + h) * n_seg + seg) * kStateFloats;
  if (seg >= n_used) {
    float4* o4 = reinterpret_cast<float4*>(out);
    for (int x = tid; x < kStateFloats / 4; x += kThreads) o4[x] = float4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  f32x4 S[kSlots][4], Z[2][2];
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[sl][nt] = zero4();
  Z[0][0] = Z[0][1] = Z[1][0] = Z[1][1] = zero4();
  Rows32 rw;
  rw.init(w, lane);
  zero_row(tl[0], tid);
  zero_row(tl[1], tid);

  // last chunk first (the sum is order-free; the walk then starts on recently read chunks),
  // one chunk in flight in registers, two LDS buffers, one barrier per chunk
  Ptrs32 p = ptrs32(pr, nullptr, k, v, b, h, (c0 + nc - 1) * C, false, tid, -1);
  Stage32 st;
  load32(st, p);
  store_state32(st, tl[0], tid);
  if (nc > 1) {
    p.next();
    load32(st, p);
  }
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    update32(tl[c & 1], rw, S, Z, w, lane, w < 4 ? w : -1);   // Z tile w on waves 0-3
    if (c + 1 < nc) store_state32(st, tl[(c + 1) & 1], tid);   // buffer read last iteration
    if (c + 2 < nc) {
      p.next();
      load32(st, p);
    }
    __syncthreads();
  }
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl) {
    if (!owns(w, sl)) continue;
    const int t = tile_of(w, sl);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      *reinterpret_cast<f32x4*>(out + ((t * 4 + nt) * 64 + lane) * 4) = S[sl][nt];
  }
  if (w < 4) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int kj = 0; kj < 2; ++kj)
        if (mi * 2 + kj == w)
          *reinterpret_cast<f32x4*>(out + kZOff + ((mi * 2 + kj) * 64 + lane) * 4) = Z[mi][kj];
  }
}

// ==========================================================================================
// Segment walk (see the file comment for the work split).  One workgroup per (segment, head,
// batch) (SegGrid).
// ==========================================================================================
struct __align__(16) Walk32Lds {
  Tiles32 tl;
  uint4 Sb[kSteps][4][64];        // S_{<c} as bf16 B operands: [K step][value tile][lane]
  uint2 Zb[4][2][64];             // Z_{<c} tiles (mi, kj) = 2 mi + kj as bf16 hi / lo A operands
  f32x4 xr[kWaves][2][64];        // readout partials handed to the other wave of a token group
  float zx[kWaves][64];           // q^T Z q halves handed to the other wave of a token group
  unsigned char dg[4 * kSteps][2];   // double group -> (a, J)
};

template <typename Tout>
__global__ __launch_bounds__(kThreads, 1) void chunk_output32_kernel(
    DevProblem pr, SegGrid sg, int L, int n_seg, const __bf16* __restrict__ q,
    const __bf16* __restrict__ k, const __bf16* __restrict__ v, Tout* __restrict__ o,
    float* __restrict__ den_out, const float* __restrict__ states, int sum_prefix) {
  extern __shared__ __align__(16) unsigned char smem[];
  Walk32Lds& sm = *reinterpret_cast<Walk32Lds*>(smem);
  Tiles32& tl = sm.tl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int tg = w & 3, ch = w >> 2;
  const SegBlock blk = seg_block(sg, pr.H);
  if (!blk.live) return;                           // padding of the grid (whole workgroup)
  const int seg = blk.seg, h = blk.h, b = blk.b;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);

  // Exclusive prefix of this segment: the scanned state at position seg, or (sum_prefix)
  // the states of segments 0 .. seg-1 added in that order; zero without states.
  f32x4 S[kSlots][4], Z[2][2];
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[sl][nt] = zero4();
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int kj = 0; kj < 2; ++kj) Z[mi][kj] = zero4();
  {
    const int j0 = sum_prefix ? 0 : seg, j1 = !states ? j0 : sum_prefix ? seg : seg + 1;
    for (int j = j0; j < j1; ++j) {
      const float* pre = states + ((long long)(b * pr.H + h) * n_seg + j) * kStateFloats;
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        if (!owns(w, sl)) continue;
        const int t = tile_of(w, sl);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          S[sl][nt] += *reinterpret_cast<const f32x4*>(pre + ((t * 4 + nt) * 64 + lane) * 4);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int kj = 0; kj < 2; ++kj)
          Z[mi][kj] += *reinterpret_cast<const f32x4*>(pre + kZOff + ((mi * 2 + kj) * 64 + lane) * 4);
    }
  }
  Rows32 rw;
  rw.init(w, lane);
  zero_row(tl, tid);
  if (tid < 4 * kSteps) {
    int a, J;
    double_group(tid, a, J);
    sm.dg[tid][0] = (unsigned char)a;
    sm.dg[tid][1] = (unsigned char)(4 * J);
  }

  // Z: wave w < 4 keeps tile (w >> 1, w & 1) and publishes it split into bf16 hi + lo
  const int zt = w < 4 ? w : -1;
  auto publish = [&]() {
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      if (!owns(w, sl)) continue;
      const int t = tile_of(w, sl);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (__bf16)S[sl][nt][r];
        reinterpret_cast<uint2*>(&sm.Sb[t >> 1][nt][lane])[t & 1] = __builtin_bit_cast(uint2, x);
      }
    }
    if (zt >= 0) {
      f32x4 zr = zero4();
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) zr = (2 * x + y == zt) ? Z[x][y] : zr;
      s16x4 zhi, zlo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const __bf16 hi = (__bf16)zr[r];
        zhi[r] = __builtin_bit_cast(short, hi);
        zlo[r] = __builtin_bit_cast(short, (__bf16)(zr[r] - (float)hi));
      }
      sm.Zb[zt][0][lane] = __builtin_bit_cast(uint2, zhi);
      sm.Zb[zt][1][lane] = __builtin_bit_cast(uint2, zlo);
    }
  };

  Ptrs32 p = ptrs32(pr, q, k, v, b, h, c0 * C, true, tid, 1);
  Stage32 st;
  load32(st, p);
  store32(st, tl, true, tid);
  publish();
  __syncthreads();

  const int t = 16 * tg + l16;                 // this lane's token (fragment column / row)
  Tout* orow = o + row_off(pr.so, b, c0 * C + 16 * tg + 8 * (lane >> 5), h) + 32 * ch + (lane & 31);
  const long long so_t = pr.so[1];

  for (int c = 0; c < nc; ++c) {
    const int tok0 = (c0 + c) * C;
    if (c + 1 < nc) {
      p.next();
      load32(st, p);
    }

    // ---- intra-chunk tile of this wave's tokens and value columns ----
    float lsum = 0.f;
    f32x4 O[2] = {zero4(), zero4()};
    const bf16x8 qf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&tl.Qs[t][8 * g]));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (2 * m > tg) break;                       // key tiles entirely in the future
      __bf16 pa[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ms = 2 * m + half;
        if (ms <= tg) {
          const bf16x8 kf = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4*>(&tl.Ks[16 * ms + l16][8 * g]));
          const f32x4 sc = mfma32(kf, qf, zero4());
          if (ms < tg)
            square_mask<false>(sc, 16 * ms, t, lane, &pa[4 * half], lsum);
          else
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
      for (int n = 0; n < 2; ++n) O[n] = mfma32(a, v_frag(tl.V, m, 2 * ch + n, lane), O[n]);
    }

    // ---- inter-chunk denominator q^T Z_{<c} q on MFMA (Z = hi + lo in bf16) ----
    // Z tile (mi, kj)'s accumulator layout is, Z being symmetric, the A operand of output rows
    // 16 kj.. and K rows 16 mi.. of y = Z q.  The two waves of a token group take the output
    // rows of kj = ch each and add their halves after the readout's exchange.
    float zq = 0.f;
    {
      s16x4 qb[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        qb[mi] = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2*>(&tl.Qs[t][16 * mi + 4 * g]));
      f32x4 y = zero4();
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        y = mfma16(__builtin_bit_cast(s16x4, sm.Zb[2 * mi + ch][0][lane]), qb[mi], y);
        y = mfma16(__builtin_bit_cast(s16x4, sm.Zb[2 * mi + ch][1][lane]), qb[mi], y);
      }
      // y[r] = (Z q_t)[16 ch + 4 g + r]
      const uint2 qq = __builtin_bit_cast(uint2, ch ? qb[1] : qb[0]);
      zq = fmaf(bf_lo(qq.x), y[0], zq);
      zq = fmaf(bf_hi(qq.x), y[1], zq);
      zq = fmaf(bf_lo(qq.y), y[2], zq);
      zq = fmaf(bf_hi(qq.y), y[3], zq);
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    zq += __shfl_xor(zq, 16);
    zq += __shfl_xor(zq, 32);
    sm.zx[w][lane] = zq;

    // ---- readout phi(q_t)^T S_{<c}: K steps [9 ch, 9 ch + 9) for all four value tiles ----
    f32x4 R[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll 3
    for (int kk = (kSteps / 2) * ch; kk < (kSteps / 2) * (ch + 1); ++kk) {
      const int ga = sm.dg[4 * kk + g][0], gj = sm.dg[4 * kk + g][1];
      const uint32_t qa = *reinterpret_cast<const uint32_t*>(&tl.Qs[t][ga]);
      const uint2 qj = *reinterpret_cast<const uint2*>(&tl.Qs[t][gj]);
      const float i0 = bf_lo(qa), i1 = bf_hi(qa);
      const float jv[4] = {bf_lo(qj.x), bf_hi(qj.x), bf_lo(qj.y), bf_hi(qj.y)};
      bf16x8 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[r] = (__bf16)(i0 * jv[r]);
        a[4 + r] = (__bf16)(i1 * jv[r]);
      }
#pragma unroll
      for (int n = 0; n < 4; ++n)
        R[n] = mfma32(a, __builtin_bit_cast(bf16x8, sm.Sb[kk][n][lane]), R[n]);
    }
    // the other wave of the token group (w ^ 4) owns the other two value tiles (selects, not
    // a runtime index, keep R in registers)
#pragma unroll
    for (int n = 0; n < 2; ++n) sm.xr[w][n][lane] = ch ? R[n] : R[2 + n];
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const f32x4 x = sm.xr[w ^ 4][n][lane], own = ch ? R[2 + n] : R[n];
#pragma unroll
      for (int r = 0; r < 4; ++r) O[n][r] += own[r] + x[r];
    }
    // both waves add the halves in the order kj = 0, 1: the same D bit for bit
    const float zo = sm.zx[w ^ 4][lane];
    const float D = pr.eps + ((ch ? zo + zq : zq + zo) + lsum);   // D_t of token t
    const float inv = 1.f / D;

    // ---- gate and store: lane holds tokens 16 tg + 4 g + r, columns 32 ch + 16 n + l16.  A
    // row-group swap between the two column tiles gives each lane a 32-column half row, so every
    // store writes whole 128-byte rows (fp32): the first register then holds tokens 16 tg + r
    // (lanes 0-31) and 16 tg + 8 + r (lanes 32-63), the second 16 tg + 4 + r and 16 tg + 12 + r.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ir = __shfl(inv, 4 * g + r);    // token 4 g + r's 1 / D (lane 4 g + r)
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(O[0][r] * ir),
                                                       __float_as_uint(O[1][r] * ir), false, false);
      // streamed out: never re-read by this kernel
      __builtin_nontemporal_store(cvt_out<Tout>(__uint_as_float(sw[0])), orow + r * so_t);
      __builtin_nontemporal_store(cvt_out<Tout>(__uint_as_float(sw[1])), orow + (4 + r) * so_t);
    }
    if (den_out && ch == 0 && lane < 16)
      den_out[((long long)b * pr.T + tok0 + t) * pr.H + h] = D;
    orow += C * so_t;

    // ---- state update with this chunk ----
    update32(tl, rw, S, Z, w, lane, zt);
    __syncthreads();                               // all reads of this chunk's tiles and Sb
    if (c + 1 < nc) {
      store32(st, tl, true, tid);
      publish();
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_chunk_state32(const DevProblem& pr, int L, int n_seg, int n_used,
                                const void* k, const void* v, float* states, hipStream_t st) {
  if (pr.p != P || pr.dv != DV || pr.C != C) return hipErrorInvalidValue;
  const size_t lds = 2 * sizeof(StateTiles32);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_state32_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const SegGrid sg = make_seg_grid(pr, n_seg);
  if (sg.blocks() > 0x7fffffffLL) return hipErrorInvalidValue;
  launch_kernel(chunk_state32_kernel, dim3((unsigned)sg.blocks()), kThreads, lds, st,
      pr, sg, L, n_seg, n_used, (const __bf16*)k, (const __bf16*)v, states);
  return hipGetLastError();
}

hipError_t launch_chunk_output32(const DevProblem& pr, bool out_bf16, int L, int n_seg,
                                 const void* q, const void* k, const void* v, void* o,
                                 float* den, const float* states, bool sum_prefix, hipStream_t st) {
  if (pr.p != P || pr.dv != DV || pr.C != C) return hipErrorInvalidValue;
  const size_t lds = sizeof(Walk32Lds);
  const SegGrid sg = make_seg_grid(pr, n_seg);
  if (sg.blocks() > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)sg.blocks());
  const __bf16 *qq = (const __bf16*)q, *kk = (const __bf16*)k, *vv = (const __bf16*)v;
  hipError_t e;
  if (out_bf16) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_output32_kernel<__bf16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    launch_kernel(chunk_output32_kernel<__bf16>, grid, kThreads, lds, st, pr, sg, L, n_seg, qq,
                  kk, vv, (__bf16*)o, den, states, (int)sum_prefix);
  } else {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_output32_kernel<float>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    launch_kernel(chunk_output32_kernel<float>, grid, kThreads, lds, st, pr, sg, L, n_seg, qq,
                  kk, vv, (float*)o, den, states, (int)sum_prefix);
  }
  return hipGetLastError();
}

}  // namespace kata

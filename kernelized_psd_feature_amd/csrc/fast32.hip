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
// state-size bullet's packed coordinates): 66 octets of 8 rows and two zero octets = 34 tiles of
// 16 rows, 17 readout K steps.  That is 140 KB of fp32 per state, too much for four waves'
// registers, so a workgroup has eight waves (two per SIMD, one workgroup per CU; waves w and
// w + 4 share a SIMD):
//   state tiles  the tiles go in K-step pairs (2 P, 2 P + 1).  Wave w owns pairs w and w + 8
//                with all four value tiles; the two tiles of the last pair go to waves 0 and 1
//                (SIMDs 0, 1) and the four Z tiles to waves 2, 3, 6, 7 (two on each of SIMDs
//                2, 3), with all four value tiles each.
//                The two tiles of a pair share their j factor rows, which the update reads
//                once, and their accumulators make whole B-operand words of the readout, which
//                the publish writes at once,
//   tokens       wave w serves tokens [16 tg, 16 tg + 16) of a chunk and the value columns
//                [32 ch, 32 ch + 32), ch = w / 4, tg = w % 4 for ch = 0 and 3 - w % 4 for
//                ch = 1: each SIMD runs token groups tg and 3 - tg, whose causal intra-chunk
//                tiles add up to the same work.  The two waves of a token group (w and 7 - w)
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
constexpr int kTiles = 34, kSteps = 17, kFull = 2;   // kFull: whole pairs per wave
constexpr int kSteps0 = (kSteps + 1) / 2;            // readout K steps of the waves with ch = 0
constexpr int kZOff = kTiles * 16 * DV;              // 34816
constexpr int kStateFloats = kZOff + 4 * 256;        // + Z as 2 x 2 tiles of 16 x 16
static_assert(kStateFloats == 34 * 16 * 64 + 4 * 256, "packed p = 32 state size (plan.h)");
constexpr int QROW = 40;                             // bf16 per q / k row: 80 B
constexpr int KTROW = 68;                            // fp32 per K^T row
constexpr int VROW = 80;                             // bf16 per v row: 160 B
// K^T rows: k_i at kt_row(i), 2 k_i at KT_D + kt_row(i), zeros at KT_Z0 and KT_Z0 + 1.  The
// row stride KTROW = 68 starts a row's 16-byte reads on bank group (row mod 8); one 8-lane
// group of the update reads k_i, 2 k_i, k_{i+2}, 2 k_{i+2} and a zero row for one parity of i,
// which this placement (doubled rows 4 groups over, the zero row of the other parity) puts on
// distinct bank groups.  kt_row rotates each block of 8 features by twice the block index:
// the staging writes of one instruction (feature 4 pc + f of 8 tokens for the pieces pc = 0-3
// or 4-7) then fall on 4 distinct bank groups too, and the reads keep their groups distinct.
constexpr int KT_D = 36, KT_Z0 = 68, KTROWS = 70;
static_assert(KT_D % 8 == 4 && KT_D >= P && KT_Z0 >= KT_D + P && KT_Z0 % 8 == 4 &&
              KTROWS == KT_Z0 + 2, "K^T row placement");
__device__ __forceinline__ int kt_row(int f) { return (f & ~7) | (((f & 7) + 2 * (f >> 3)) & 7); }

// q row t starts 8 bytes in when t mod 16 >= 8: the readout's 4- and 8-byte reads of 16
// consecutive tokens then fall on distinct banks (the 80-byte pitch alone repeats every 8
// rows); the 32 values stay inside the 40-value row.  Reads of q rows are 8 bytes or less.
__device__ __forceinline__ int q_skew(int t) { return 4 * ((t >> 3) & 1); }
static_assert(QROW >= P + 4, "q row skew");

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

// Tile ownership (see the file comment): whole pair ps < kFull of wave w, the tile 32 + e of
// the last pair (e >= 0 on waves 0, 1) and the Z tile index (z >= 0 on waves 2, 3, 6, 7).
__host__ __device__ constexpr int pair_of(int w, int ps) { return w + 8 * ps; }
__host__ __device__ constexpr int extra_of(int w) { return w < 2 ? w : -1; }
__host__ __device__ constexpr int ztile_of(int w) { return (w & 2) ? (w & 1) + 2 * (w >> 2) : -1; }
// token group of wave w (see the file comment); its partner wave is 7 - w
__device__ __forceinline__ int tgroup_of(int w) { return w < 4 ? w : 7 - w; }
static_assert(2 * (8 * kFull + 1) == kTiles, "pairs: kFull per wave and one split pair");
// one extra 16 x 64 tile per wave at most (the last pair's or a Z tile), so one accumulator set
static_assert(extra_of(0) == 0 && extra_of(1) == 1 && ztile_of(2) == 0 && ztile_of(3) == 1 &&
              ztile_of(6) == 2 && ztile_of(7) == 3 && extra_of(4) < 0 && ztile_of(5) < 0,
              "tile ownership");

// Row order of the packed state.  K step kk covers tiles 2 kk and 2 kk + 1; its octet g (the
// readout's lane group g = lane / 16) is rows 4 g + r of both tiles, r = 0..3, the readout's
// K slots r and 4 + r of the lane.  The two rows of a slot pair share their second feature
// j(r), so the update reads one j factor row for both.  Octet kinds (x = the features
// 4 J .. 4 J + 3 of column block J):
//   R (a, J)  off the diagonal blocks, a even, a + 1 < 4 J: rows (a, 4 J + r), (a + 1, 4 J + r),
//   D J       the diagonal block J: rows (x_r, x_r) and (x_{3, 2, 3, 1 [r]}, x_r),
//   L B       the pairs (x_1, x_0) and (x_2, x_0) of block B + r, the two that D J leaves out,
//   zero      two octets of zero rows (528 = 66 x 8 pairs, 17 K steps hold 68 octets).
// Steps: plain R (a = a0 + 2 g, J = J0); split R (lane groups 0, 1: a = a0 + 2 g in block J0,
// lane groups 2, 3: a = a0 + 2 (g - 2) in block J0 + 2; the column blocks J = 1, 3, 5, 7 have
// 2 J = 2 mod 4 octets R); D (J = J0 + g); and the last step, L (B = 4 g) in lane groups 0, 1
// and zero octets in lane groups 2, 3.  Every lane group of a step reads its q values at one
// lane offset plus a constant, and consecutive R steps of one column block share their j.
enum { kPlainR = 0, kSplitR = 1, kDiag = 2, kLeft = 3 };
struct Step32 {
  int kind, a0, J0;
};
// 3-bit fields per step (low step first): J0 and a0 / 4; shifts, not a table in memory, so a
// runtime kk (the update's row set-up) costs no private memory
constexpr uint64_t pack3(const int (&f)[kSteps], int div) {
  uint64_t x = 0;
  for (int i = kSteps - 1; i >= 0; --i) x = (x << 3) | uint64_t(f[i] / div);
  return x;
}
constexpr int kStepJ0[kSteps] = {1, 2, 3, 4, 4, 5, 5, 5, 6, 6, 6, 7, 7, 7, 0, 4, 0};
constexpr int kStepA0[kSteps] = {0, 0, 4, 0, 8, 0, 4, 12, 0, 8, 16, 4, 12, 20, 0, 0, 0};
constexpr uint64_t kJ0Bits = pack3(kStepJ0, 1), kA0Bits = pack3(kStepA0, 4);
__host__ __device__ constexpr Step32 step32(int kk) {
  const int kind = kk == 0 || kk == 5 ? kSplitR : kk == 14 || kk == 15 ? kDiag
                 : kk == 16 ? kLeft : kPlainR;
  return Step32{kind, 4 * int((kA0Bits >> (3 * kk)) & 7), int((kJ0Bits >> (3 * kk)) & 7)};
}
// second feature of D J's rows 4 + r (the first rows are the squares)
__host__ __device__ constexpr int diag_i(int r) { return r == 1 ? 2 : r == 3 ? 1 : 3; }
// Features (i, j) of row 4 g + r of tile 2 kk + tp; i < 0 for a zero row.
__host__ __device__ constexpr void row32(int kk, int g, int r, int tp, int& i, int& j) {
  const Step32 s = step32(kk);
  if (s.kind == kPlainR || s.kind == kSplitR) {
    const int a = s.kind == kSplitR ? s.a0 + 2 * (g & 1) : s.a0 + 2 * g;
    const int J = s.kind == kSplitR ? s.J0 + 2 * (g >> 1) : s.J0;
    i = a + tp;
    j = 4 * J + r;
  } else if (s.kind == kDiag) {
    const int x = 4 * (s.J0 + g);
    i = tp ? x + diag_i(r) : x + r;
    j = x + r;
  } else if (g < 2) {
    const int x = 4 * (4 * g + r);
    i = x + 1 + tp;
    j = x;
  } else {
    i = -1;
    j = 0;
  }
}
// every unordered pair of the 32 features exactly once, 16 zero rows, and one j per slot pair
constexpr bool rows32_cover() {
  int seen[32][32] = {};
  int zeros = 0;
  for (int kk = 0; kk < kSteps; ++kk)
    for (int g = 0; g < 4; ++g)
      for (int r = 0; r < 4; ++r) {
        int j0 = 0;
        for (int tp = 0; tp < 2; ++tp) {
          int i = 0, j = 0;
          row32(kk, g, r, tp, i, j);
          if (tp == 0) j0 = j;
          if (i < 0) {
            ++zeros;
            continue;
          }
          if (i > 31 || j < 0 || j > 31 || j != j0) return false;
          if (seen[i < j ? i : j][i < j ? j : i]++) return false;
        }
      }
  for (int i = 0; i < 32; ++i)
    for (int j = i; j < 32; ++j)
      if (seen[i][j] != 1) return false;
  return zeros == 16;
}
static_assert(rows32_cover(), "p = 32 packed row order");

// One thread's share of a chunk's loads: 8 bytes (features 4 pc .. 4 pc + 3) of the q row
// and of the k row of token stage_row, and 16 bytes of one v row (row tid / 8, columns
// 8 (tid % 8) ..).  Wave w stages tokens 8 w .. 8 w + 7; lanes 0-31 hold features 0-15 and
// lanes 32-63 features 16-31, so one K^T store instruction (feature 4 pc + f of 8 tokens for
// 4 pieces pc) falls on 4 distinct bank groups (kt_row) and every thread stores the same share.
__device__ __forceinline__ int stage_row(int tid) { return 8 * (tid >> 6) + ((tid & 31) >> 2); }
__device__ __forceinline__ int stage_piece(int tid) { return 4 * ((tid >> 5) & 1) + (tid & 3); }

struct Stage32 {
  uint2 q, k;
  uint4 v;
};

struct Ptrs32 {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  long long q_step, k_step, v_step;
  __device__ __forceinline__ void next() {
    if (q) q += q_step;
    k += k_step;
    v += v_step;
  }
};

__device__ __forceinline__ Ptrs32 ptrs32(const DevProblem& pr, const __bf16* q, const __bf16* k,
                                         const __bf16* v, int b, int h, int tok0, bool with_q,
                                         int tid, int dir) {
  Ptrs32 p;
  const int row = stage_row(tid), pc = stage_piece(tid);
  p.q = with_q ? q + row_off(pr.sq, b, tok0 + row, h) + 4 * pc : nullptr;
  p.q_step = (long long)dir * C * pr.sq[1];
  p.k = k + row_off(pr.sk, b, tok0 + row, h) + 4 * pc;
  p.k_step = (long long)dir * C * pr.sk[1];
  p.v = v + row_off(pr.sv, b, tok0 + (tid >> 3), h) + 8 * (tid & 7);
  p.v_step = (long long)dir * C * pr.sv[1];
  return p;
}

__device__ __forceinline__ void load32(Stage32& s, const Ptrs32& p) {
  if (p.q) s.q = *reinterpret_cast<const uint2*>(p.q);
  s.k = *reinterpret_cast<const uint2*>(p.k);
  s.v = ld16(p.v);
}

// k piece -> K^T rows (k, 2 k)
template <class TL>
__device__ __forceinline__ void store_kt(const Stage32& s, TL& tl, int tid) {
  const int row = stage_row(tid), pc = stage_piece(tid);
  const uint32_t wd[2] = {s.k.x, s.k.y};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float a = bf_lo(wd[e]), c = bf_hi(wd[e]);
    const int ra = kt_row(4 * pc + 2 * e), rc = kt_row(4 * pc + 2 * e + 1);
    tl.KT[ra][row] = a;
    tl.KT[rc][row] = c;
    tl.KT[KT_D + ra][row] = 2.f * a;        // exact
    tl.KT[KT_D + rc][row] = 2.f * c;
  }
}

// q / k pieces -> row-major rows (q when the tile has them) and K^T rows; v piece -> V
__device__ __forceinline__ void store32(const Stage32& s, Tiles32& tl, bool with_q, int tid) {
  const int row = stage_row(tid), pc = stage_piece(tid);
  if (with_q) *reinterpret_cast<uint2*>(&tl.Qs[row][q_skew(row) + 4 * pc]) = s.q;
  *reinterpret_cast<uint2*>(&tl.Ks[row][4 * pc]) = s.k;
  store_kt(s, tl, tid);
  *reinterpret_cast<uint4*>(&tl.V[tid >> 3][8 * (tid & 7)]) = s.v;
}

__device__ __forceinline__ void store_state32(const Stage32& s, StateTiles32& tl, int tid) {
  store_kt(s, tl, tid);
  *reinterpret_cast<uint4*>(&tl.V[tid >> 3][8 * (tid & 7)]) = s.v;
}

template <class TL>
__device__ __forceinline__ void zero_row(TL& tl, int tid) {
  if (tid < 2 * KTROW) tl.KT[KT_Z0 + tid / KTROW][tid % KTROW] = 0.f;
}

// A operands of the packed update for this lane's row of the two tiles of a pair (irow[tp]
// selects k_i, 2 k_i or zeros; the pair shares the j row), 32-key step m in slot order kappa.
template <class TL>
__device__ __forceinline__ void phik2(const TL& tl, const int (&irow)[2], int jrow, int m,
                                      int lane, bf16x8 (&a)[2]) {
  const int g = lane >> 4;
  const float4 ja = *reinterpret_cast<const float4*>(&tl.KT[jrow][32 * m + 4 * g]);
  const float4 jb = *reinterpret_cast<const float4*>(&tl.KT[jrow][32 * m + 16 + 4 * g]);
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    const float4 ia = *reinterpret_cast<const float4*>(&tl.KT[irow[tp]][32 * m + 4 * g]);
    const float4 ib = *reinterpret_cast<const float4*>(&tl.KT[irow[tp]][32 * m + 16 + 4 * g]);
    const uint4 f{pack_bf16x2(ia.x * ja.x, ia.y * ja.y), pack_bf16x2(ia.z * ja.z, ia.w * ja.w),
                  pack_bf16x2(ib.x * jb.x, ib.y * jb.y), pack_bf16x2(ib.z * jb.z, ib.w * jb.w)};
    a[tp] = __builtin_bit_cast(bf16x8, f);
  }
}

// k_s[16 mi + lane%16] over the slots of 32-key step m (operand of Z = K^T K)
template <class TL>
__device__ __forceinline__ bf16x8 kcol(const TL& tl, int mi, int m, int lane) {
  const int i = kt_row(16 * mi + (lane & 15)), g = lane >> 4;
  const float4 a = *reinterpret_cast<const float4*>(&tl.KT[i][32 * m + 4 * g]);
  const float4 c = *reinterpret_cast<const float4*>(&tl.KT[i][32 * m + 16 + 4 * g]);
  bf16x8 f;
  f[0] = (__bf16)a.x; f[1] = (__bf16)a.y; f[2] = (__bf16)a.z; f[3] = (__bf16)a.w;
  f[4] = (__bf16)c.x; f[5] = (__bf16)c.y; f[6] = (__bf16)c.z; f[7] = (__bf16)c.w;
  return f;
}

// Row sources of this lane's row of each owned pair: ps < kFull the whole pairs, ps = kFull
// the last pair (its tile 32 + e in irow[kFull][0], when the wave has one).
struct Rows32 {
  int irow[kFull + 1][2], jrow[kFull + 1];
  __device__ void init(int w, int e, int lane) {
#pragma unroll
    for (int ps = 0; ps <= kFull; ++ps) {
      const int P = ps < kFull ? pair_of(w, ps) : 16, row = lane & 15;
      int j = 0;
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        int i = 0;
        row32(P, row >> 2, row & 3, ps < kFull ? tp : max(e, 0), i, j);   // j: the same for both
        irow[ps][tp] = i < 0 ? KT_Z0 + (row & 1) : (i == j ? kt_row(i) : KT_D + kt_row(i));
      }
      jrow[ps] = kt_row(j);
    }
  }
};

// The accumulators of one wave's share of S and Z: S[ps][tp][nt] for tile 2 pair_of(w, ps) + tp
// and value tile nt; X[nt] for tile 32 + e and value tile nt (e >= 0), or X[0] for the Z tile
// (z >> 1, z & 1) (z >= 0).
struct Acc32 {
  f32x4 S[kFull][2][4];
  f32x4 X[4];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int ps = 0; ps < kFull; ++ps)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) S[ps][tp][nt] = zero4();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) X[nt] = zero4();
  }
  // f(accumulator, state float offset of its fragment) for every owned fragment
  template <class F>
  __device__ __forceinline__ void each(int w, int e, int z, int lane, F&& f) {
#pragma unroll
    for (int ps = 0; ps < kFull; ++ps)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          f(S[ps][tp][nt], (((2 * pair_of(w, ps) + tp) * 4 + nt) * 64 + lane) * 4);
    if (e >= 0) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) f(X[nt], (((32 + e) * 4 + nt) * 64 + lane) * 4);
    }
    if (z >= 0) f(X[0], kZOff + (z * 64 + lane) * 4);
  }
};

// S += Phi(K)^T V over one staged chunk; the Z accumulator += the 16 x 16 tile (z >> 1, z & 1)
// of K^T K when z >= 0.  e and z are wave-uniform.
template <class TL>
__device__ __forceinline__ void update32(const TL& tl, const Rows32& rw, Acc32& acc, int e,
                                         int lane, int z) {
  // both 32-key steps unrolled: the LDS addresses of the second become immediate offsets
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    bf16x8 vb[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) vb[nt] = v_frag(tl.V, m, nt, lane);
#pragma unroll
    for (int ps = 0; ps < kFull; ++ps) {
      bf16x8 a[2];
      phik2(tl, rw.irow[ps], rw.jrow[ps], m, lane, a);
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc.S[ps][tp][nt] = mfma32(a[tp], vb[nt], acc.S[ps][tp][nt]);
    }
    if (e >= 0) {                    // tile 32 + e, all four value tiles
      const int g = lane >> 4, ir = rw.irow[kFull][0], jr = rw.jrow[kFull];
      const float4 ja = *reinterpret_cast<const float4*>(&tl.KT[jr][32 * m + 4 * g]);
      const float4 jb = *reinterpret_cast<const float4*>(&tl.KT[jr][32 * m + 16 + 4 * g]);
      const float4 ia = *reinterpret_cast<const float4*>(&tl.KT[ir][32 * m + 4 * g]);
      const float4 ib = *reinterpret_cast<const float4*>(&tl.KT[ir][32 * m + 16 + 4 * g]);
      const uint4 f{pack_bf16x2(ia.x * ja.x, ia.y * ja.y), pack_bf16x2(ia.z * ja.z, ia.w * ja.w),
                    pack_bf16x2(ib.x * jb.x, ib.y * jb.y), pack_bf16x2(ib.z * jb.z, ib.w * jb.w)};
      const bf16x8 a = __builtin_bit_cast(bf16x8, f);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc.X[nt] = mfma32(a, vb[nt], acc.X[nt]);
    }
    if (z >= 0) {
      const int mi = z >> 1, kj = z & 1;
      const bf16x8 a = kcol(tl, mi, m, lane), bb = kcol(tl, kj, m, lane);
      acc.X[0] = mfma32(a, bb, acc.X[0]);
    }
  }
}

// ==========================================================================================
// Segment state: S_seg = sum over the segment's chunks of Phi(K_c)^T V_c, Z_seg = sum K^T K.
// One workgroup per (segment, head, batch) (SegGrid).  sp == 0: workgroup seg sums segment
// seg into state seg; segments seg >= n_used get a zero state without reading their tokens.
// sp > 0 (spread): workgroup u sums the chunks [u sp, min((u + 1) sp, (n_seg - 1) L)), first to
// last, into state 2 u: the whole range, or, when the range crosses a segment boundary (sp <=
// L: at most one), the chunks before it, and then state 2 u + 1 the whole range.  Empty ranges
// write nothing.
// State layout (floats): tile t, value tile nt, lane -> ((t * 4 + nt) * 64 + lane) * 4, then
// Z tile (mi, kj) -> kZOff + ((mi * 2 + kj) * 64 + lane) * 4.
// ==========================================================================================
__global__ __launch_bounds__(kThreads, 1) void chunk_state32_kernel(
    DevProblem pr, SegGrid sg, int L, int n_seg, int n_used, int sp, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, float* __restrict__ states) {
  extern __shared__ __align__(16) unsigned char smem[];
  StateTiles32* tl = reinterpret_cast<StateTiles32*>(smem);    // two buffers
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = extra_of(w), z = ztile_of(w);
  const SegBlock blk = seg_block(sg, pr.H);
  if (!blk.live) return;                           // padding of the grid (whole workgroup)
  const int seg = blk.seg, h = blk.h, b = blk.b;
  const int n_chunks = pr.T / C;
  const long long seq = (long long)b * pr.H + h;
  int c0, nc, flush = -1;          // chunk range; iteration that first sums a chunk past the boundary
  float *out, *out_all = nullptr;   // spread and crossing: the part before the boundary, the whole
  if (sp == 0) {
    c0 = seg * L;
    nc = min(L, n_chunks - c0);
    out = states + (seq * n_seg + seg) * kStateFloats;
    if (seg >= n_used) {
      float4* o4 = reinterpret_cast<float4*>(out);
      for (int x = tid; x < kStateFloats / 4; x += kThreads) o4[x] = float4{0.f, 0.f, 0.f, 0.f};
      return;
    }
  } else {
    c0 = seg * sp;
    nc = min(sp, (n_seg - 1) * L - c0);
    if (nc <= 0) return;
    out = states + (seq * n_seg + seg) * 2 * kStateFloats;
    const int bnd = (c0 / L + 1) * L;
    if (bnd < c0 + nc) {
      out_all = out + kStateFloats;
      flush = bnd - c0;              // chunks are summed first to last
    }
  }
  Acc32 acc;
  acc.zero();
  Rows32 rw;
  rw.init(w, e, lane);
  zero_row(tl[0], tid);
  zero_row(tl[1], tid);

  // one state per segment: last chunk first (the walk then starts on recently read chunks);
  // spread: first to last, so the sum at the boundary is the part before it.  Two chunks in
  // flight in registers (one workgroup per CU: no other workgroup hides their latency), two
  // LDS buffers, one barrier per chunk.
  const int dir = sp == 0 ? -1 : 1;
  Ptrs32 p = ptrs32(pr, nullptr, k, v, b, h, (dir < 0 ? c0 + nc - 1 : c0) * C, false, tid, dir);
  Stage32 sa, sb;
  load32(sa, p);
  store_state32(sa, tl[0], tid);
  if (nc > 1) {                      // chunk 1
    p.next();
    load32(sa, p);
  }
  if (nc > 2) {                      // chunk 2
    p.next();
    load32(sb, p);
  }
  __syncthreads();
  auto emit = [&](float* dst) {
    acc.each(w, e, z, lane, [&](f32x4& x, int off) { *reinterpret_cast<f32x4*>(dst + off) = x; });
  };
  // chunk c from LDS; `nx` holds chunk c + 1, which goes to the other buffer (read in the
  // previous iteration, before its barrier), and then takes chunk c + 3
  auto step = [&](int c, Stage32& nx) {
    if (c == flush) emit(out);       // the chunks before the segment boundary
    update32(tl[c & 1], rw, acc, e, lane, z);
    if (c + 1 < nc) store_state32(nx, tl[(c + 1) & 1], tid);
    if (c + 3 < nc) {
      p.next();
      load32(nx, p);
    }
    __syncthreads();
  };
  for (int c = 0; c < nc; c += 2) {
    step(c, sa);
    if (c + 1 < nc) step(c + 1, sb);
  }
  emit(out_all ? out_all : out);
}

struct Pair4 {
  f32x4 a, b;
};

// The intra-chunk tile of wave w's tokens and value columns (the walk's first product), for a
// chunk whose values hold an infinity or a nan: the step holding the diagonal tile (and any
// future keys) takes finite_or_zero value operands and nonfinite_fixup adds the exact
// contributions of the non-finite values of unmasked pairs, so no later token reaches an
// earlier output.  Not inlined: the walk's loop keeps its registers and schedule, and only
// this rare path pays for the call.
__device__ __attribute__((noinline)) Pair4 intra_exact32(const Tiles32& tl, bf16x8 qf, int w,
                                                         int lane) {
  const int g = lane >> 4, l16 = lane & 15, tg = tgroup_of(w), ch = w >> 2, t = 16 * tg + l16;
  float lsum = 0.f;
  f32x4 O[2] = {zero4(), zero4()};
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (2 * m > tg) break;
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
    if (2 * m + 1 < tg) {                          // keys before every token of the wave
#pragma unroll
      for (int n = 0; n < 2; ++n) O[n] = mfma32(a, v_frag(tl.V, m, 2 * ch + n, lane), O[n]);
    } else {
#pragma unroll
      for (int n = 0; n < 2; ++n)
        O[n] = mfma32(a, finite_or_zero(v_frag(tl.V, m, 2 * ch + n, lane)), O[n]);
      const int cols[2] = {32 * ch + l16, 32 * ch + 16 + l16};
      nonfinite_fixup<2>(O, tl.V, a, 32 * m, 16 * tg, cols, lane);
    }
  }
  return Pair4{O[0], O[1]};
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
  float inv[kWaves][16];          // per wave: 1 / D_t of its token group's 16 tokens
  uint32_t vbad[kWaves];          // per wave: its staged v row pieces hold a non-finite value
};

// One readout K step's LDS operands: this lane's q words (the fields its step kind uses) and
// the four B-operand words of the state.
struct RdOps32 {
  uint32_t qi;
  uint2 qv;
  uint4 u0, u1;
  uint4 sb[4];
};
template <int KK, bool kLoadJ = true>
__device__ __forceinline__ void rd_load32(RdOps32& o, const uint4 (*Sb)[4][64],
                                          const __bf16* const (&qa)[2], const __bf16* const (&qj)[2],
                                          const __bf16* qd, const __bf16* ql, int lane) {
  constexpr Step32 st = step32(KK);
  if constexpr (st.kind == kPlainR || st.kind == kSplitR) {
    o.qi = *reinterpret_cast<const uint32_t*>(qa[st.kind] + st.a0);
    if constexpr (kLoadJ) o.qv = *reinterpret_cast<const uint2*>(qj[st.kind] + 4 * st.J0);
  } else if constexpr (st.kind == kDiag) {
    o.qv = *reinterpret_cast<const uint2*>(qd + 4 * st.J0);
  } else {
    const uint2 h0 = *reinterpret_cast<const uint2*>(ql), h1 = *reinterpret_cast<const uint2*>(ql + 4);
    const uint2 h2 = *reinterpret_cast<const uint2*>(ql + 8), h3 = *reinterpret_cast<const uint2*>(ql + 12);
    o.u0 = uint4{h0.x, h0.y, h1.x, h1.y};
    o.u1 = uint4{h2.x, h2.y, h3.x, h3.y};
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) o.sb[n] = Sb[KK][n][lane];
}
template <int KK>
__device__ __forceinline__ void rd_step32(const RdOps32& o, f32x4 (&R)[4]) {
  constexpr Step32 st = step32(KK);
  float x[8], y[8];                   // slot s of the A operand is x[s] * y[s]
  if constexpr (st.kind == kPlainR || st.kind == kSplitR) {
    const float jv[4] = {bf_lo(o.qv.x), bf_hi(o.qv.x), bf_lo(o.qv.y), bf_hi(o.qv.y)};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = bf_lo(o.qi);
      x[4 + r] = bf_hi(o.qi);
      y[r] = y[4 + r] = jv[r];
    }
  } else if constexpr (st.kind == kDiag) {
    const float xv[4] = {bf_lo(o.qv.x), bf_hi(o.qv.x), bf_lo(o.qv.y), bf_hi(o.qv.y)};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = xv[r];
      x[4 + r] = xv[diag_i(r)];
      y[r] = y[4 + r] = xv[r];
    }
  } else {
    // blocks 4 (g & 1) + r: x_0, x_1 in the low word of the block, x_2 in the high one
    const uint32_t w01[4] = {o.u0.x, o.u0.z, o.u1.x, o.u1.z};
    const uint32_t w23[4] = {o.u0.y, o.u0.w, o.u1.y, o.u1.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x0 = bf_lo(w01[r]);
      x[r] = bf_hi(w01[r]);
      x[4 + r] = bf_lo(w23[r]);
      y[r] = y[4 + r] = x0;
    }
  }
  bf16x8 a;
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) a[sl] = (__bf16)(x[sl] * y[sl]);
#pragma unroll
  for (int n = 0; n < 4; ++n) R[n] = mfma32(a, __builtin_bit_cast(bf16x8, o.sb[n]), R[n]);
}
// Steps KK .. K1 - 1, the operands of KK already in cur: the next step's loads are issued
// before this step's arithmetic (a scheduling barrier keeps them there), so their LDS latency
// hides behind it.  Consecutive plain R steps of one column block take their j quad from the
// previous step (the barrier would otherwise keep the compiler from sharing it).
template <int KK, int K1>
__device__ __forceinline__ void rd_steps32(const RdOps32& cur, const uint4 (*Sb)[4][64],
                                           const __bf16* const (&qa)[2],
                                           const __bf16* const (&qj)[2], const __bf16* qd,
                                           const __bf16* ql, int lane, f32x4 (&R)[4]) {
  if constexpr (KK + 1 < K1) {
    constexpr Step32 a = step32(KK), b = step32(KK + 1);
    constexpr bool same_j = a.kind == kPlainR && b.kind == kPlainR && a.J0 == b.J0;
    RdOps32 nxt;
    rd_load32<KK + 1, !same_j>(nxt, Sb, qa, qj, qd, ql, lane);
    if constexpr (same_j) nxt.qv = cur.qv;
    __builtin_amdgcn_sched_barrier(0);
    rd_step32<KK>(cur, R);
    rd_steps32<KK + 1, K1>(nxt, Sb, qa, qj, qd, ql, lane, R);
  } else {
    rd_step32<KK>(cur, R);
  }
}

// Readout phi(q_t)^T S_{<c} over the K steps [kSteps0 CH, ..) of the waves with ch = CH, for all
// four value tiles.  qa, qj, qd and ql point into this lane's q row at the lane offsets of the
// step kinds (R plain / split: the i pair and the j quad; D: the block; L: the four blocks),
// so each step's loads take constant offsets from them.
template <int CH>
__device__ __forceinline__ void readout32(const uint4 (*Sb)[4][64], const __bf16* const (&qa)[2],
                                          const __bf16* const (&qj)[2], const __bf16* qd,
                                          const __bf16* ql, int lane, f32x4 (&R)[4]) {
  constexpr int k0 = CH ? kSteps0 : 0, k1 = CH ? kSteps : kSteps0;
  RdOps32 first;
  rd_load32<k0>(first, Sb, qa, qj, qd, ql, lane);
  rd_steps32<k0, k1>(first, Sb, qa, qj, qd, ql, lane, R);
}

template <typename Tout>
__global__ __launch_bounds__(kThreads, 1) void chunk_output32_kernel(
    DevProblem pr, SegGrid sg, int L, int n_seg, int sp, const __bf16* __restrict__ q,
    const __bf16* __restrict__ k, const __bf16* __restrict__ v, Tout* __restrict__ o,
    float* __restrict__ den_out, const float* __restrict__ states, int sum_prefix) {
  extern __shared__ __align__(16) unsigned char smem[];
  Walk32Lds& sm = *reinterpret_cast<Walk32Lds*>(smem);
  Tiles32& tl = sm.tl;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tg = tgroup_of(w), ch = w >> 2;
  const SegBlock blk = seg_block(sg, pr.H);
  if (!blk.live) return;                           // padding of the grid (whole workgroup)
  const int seg = blk.seg, h = blk.h, b = blk.b;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);

  // Exclusive prefix of this segment: the scanned state at position seg, or (sum_prefix)
  // the states of segments 0 .. seg-1 added in that order, or (sp > 0) the sums of the spread
  // state pass over the chunks before seg L, in the order of their ranges (a range that ends
  // by seg L: its whole sum; the range that crosses seg L: its part before it); zero without
  // states.
  // Z: wave w with zt >= 0 keeps tile (zt >> 1, zt & 1) in acc.X[0] and publishes it split into
  // bf16 hi + lo.
  const int e = extra_of(w), zt = ztile_of(w);
  Acc32 acc;
  acc.zero();
  {
    auto add = [&](const float* pre) {
      acc.each(w, e, zt, lane, [&](f32x4& x, int off) { x += *reinterpret_cast<const f32x4*>(pre + off); });
    };
    const long long seq = (long long)b * pr.H + h;
    if (states && sp > 0) {
      for (int u = 0; u < n_seg; ++u) {
        const int lo = u * sp, hi = min(lo + sp, (n_seg - 1) * L), bnd = (lo / L + 1) * L;
        if (lo >= hi || lo >= seg * L) break;        // ranges ascend
        const float* pre = states + (seq * n_seg + u) * 2 * kStateFloats;
        // crossing a boundary: state 2 u is [lo, bnd), 2 u + 1 the whole range; else 2 u
        add(bnd < hi && hi <= seg * L ? pre + kStateFloats : pre);
      }
    } else {
      const int j0 = sum_prefix ? 0 : seg, j1 = !states ? j0 : sum_prefix ? seg : seg + 1;
      for (int j = j0; j < j1; ++j) add(states + (seq * n_seg + j) * kStateFloats);
    }
  }
  Rows32 rw;
  rw.init(w, e, lane);
  zero_row(tl, tid);

  // a pair's two accumulators -> one B-operand word of its K step (tile 2 P in the low half)
  auto bword = [](const f32x4& lo, const f32x4& hi) {
    return uint4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                 pack_bf16x2(hi[2], hi[3])};
  };
  auto publish = [&]() {
#pragma unroll
    for (int ps = 0; ps < kFull; ++ps)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        sm.Sb[pair_of(w, ps)][nt][lane] = bword(acc.S[ps][0][nt], acc.S[ps][1][nt]);
    if (e >= 0) {                    // tile 32 + e: half e of the last K step's words
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        reinterpret_cast<uint2*>(&sm.Sb[16][nt][lane])[e] =
            uint2{pack_bf16x2(acc.X[nt][0], acc.X[nt][1]), pack_bf16x2(acc.X[nt][2], acc.X[nt][3])};
    }
    if (zt >= 0) {
      const f32x4 zr = acc.X[0];
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

  // Each wave records whether the v pieces it stages hold an infinity or a nan; the chunk's
  // masked P.V step then takes the slow exact path (nonfinite_fixup in mfma_util.h).
  auto flag_v = [&](const Stage32& x) {
    const uint32_t any = __any(nonfinite_bf16x8(x.v) != 0u) ? 1u : 0u;
    if (lane == 0) sm.vbad[w] = any;
  };

  Ptrs32 p = ptrs32(pr, q, k, v, b, h, c0 * C, true, tid, 1);
  Stage32 st;
  load32(st, p);
  store32(st, tl, true, tid);
  flag_v(st);
  publish();
  __syncthreads();

  const int t = 16 * tg + l16;                 // this lane's token (fragment column / row)
  const __bf16* const qrow = &tl.Qs[t][q_skew(t)];
  const __bf16* const qa[2] = {qrow + 2 * g, qrow + 2 * (g & 1)};
  const __bf16* const qj[2] = {qrow, qrow + 8 * (g >> 1)};
  const __bf16* const qd = qrow + 4 * g;
  const __bf16* const ql = qrow + 16 * (g & 1);
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
    const uint2 qf0 = *reinterpret_cast<const uint2*>(qrow + 8 * g);
    const uint2 qf1 = *reinterpret_cast<const uint2*>(qrow + 8 * g + 4);
    const bf16x8 qf = __builtin_bit_cast(bf16x8, uint4{qf0.x, qf0.y, qf1.x, qf1.y});
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (2 * m > tg) break;                       // key tiles entirely in the future
      uint32_t pw[2][2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ms = 2 * m + half;
        if (ms <= tg) {
          const bf16x8 kf = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4*>(&tl.Ks[16 * ms + l16][8 * g]));
          const f32x4 sc = mfma32(kf, qf, zero4());
          f32x4 x2;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // the diagonal tile (ms == tg): keys 16 tg + 4 g + r against token 16 tg + l16; one
            // select whose condition folds the wave-uniform tile test into the lane mask
            x2[r] = (ms < tg || 4 * g + r <= l16) ? sc[r] * sc[r] : 0.f;
          }
          // bf16 weights in pairs, their row sum from the same rounded values (v_dot2 with ones)
          pw[half][0] = pack_bf16x2(x2[0], x2[1]);
          pw[half][1] = pack_bf16x2(x2[2], x2[3]);
          lsum = sum_bf16x2(pw[half][0], lsum);
          lsum = sum_bf16x2(pw[half][1], lsum);
        } else {
          pw[half][0] = pw[half][1] = 0u;
        }
      }
      const bf16x8 a = __builtin_bit_cast(bf16x8, uint4{pw[0][0], pw[0][1], pw[1][0], pw[1][1]});
#pragma unroll
      for (int n = 0; n < 2; ++n) O[n] = mfma32(a, v_frag(tl.V, m, 2 * ch + n, lane), O[n]);
    }
    {
      // a value of the chunk is an infinity or a nan (rare): the tile again, exactly
      const uint4 vb0 = *reinterpret_cast<const uint4*>(&sm.vbad[0]);
      const uint4 vb1 = *reinterpret_cast<const uint4*>(&sm.vbad[4]);
      if (__builtin_amdgcn_readfirstlane(vb0.x | vb0.y | vb0.z | vb0.w | vb1.x | vb1.y | vb1.z |
                                         vb1.w) != 0) {
        const Pair4 e = intra_exact32(tl, qf, w, lane);
        O[0] = e.a;
        O[1] = e.b;
      }
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
        qb[mi] = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2*>(qrow + 16 * mi + 4 * g));
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
    lsum = sum_xor32(sum_xor16(lsum));
    zq = sum_xor32(sum_xor16(zq));
    sm.zx[w][lane] = zq;

    // ---- readout phi(q_t)^T S_{<c}: the first kSteps0 K steps (ch = 0) or the rest (ch = 1) ----
    f32x4 R[4] = {zero4(), zero4(), zero4(), zero4()};
    if (ch)
      readout32<1>(sm.Sb, qa, qj, qd, ql, lane, R);
    else
      readout32<0>(sm.Sb, qa, qj, qd, ql, lane, R);
    // the other wave of the token group (7 - w) owns the other two value tiles (selects, not
    // a runtime index, keep R in registers); it reads them after the update's barrier
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      sm.xr[w][n][lane] = ch ? R[n] : R[2 + n];
      const f32x4 own = ch ? R[2 + n] : R[n];
#pragma unroll
      for (int r = 0; r < 4; ++r) O[n][r] += own[r];
    }

    // ---- state update with this chunk (registers only: Sb keeps S_{<c} until the barrier) ----
    update32(tl, rw, acc, e, lane, zt);
    __syncthreads();          // all reads of this chunk's tiles, Sb and Zb; xr and zx written
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const f32x4 x = sm.xr[7 - w][n][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) O[n][r] += x[r];
    }
    // both waves add the halves in the order kj = 0, 1: the same D bit for bit
    const float zo = sm.zx[7 - w][lane];
    const float D = pr.eps + ((ch ? zo + zq : zq + zo) + lsum);   // D_t of token t
    if (g == 0) sm.inv[w][l16] = __builtin_amdgcn_rcpf(D);        // 1 ulp
    const float4 inv4 = *reinterpret_cast<const float4*>(&sm.inv[w][4 * g]);   // own writes
    const float invr[4] = {inv4.x, inv4.y, inv4.z, inv4.w};

    // ---- gate and store: lane holds tokens 16 tg + 4 g + r, columns 32 ch + 16 n + l16.  A
    // row-group swap between the two column tiles gives each lane a 32-column half row, so every
    // store writes whole 128-byte rows (fp32): the first register then holds tokens 16 tg + r
    // (lanes 0-31) and 16 tg + 8 + r (lanes 32-63), the second 16 tg + 4 + r and 16 tg + 12 + r.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ir = invr[r];                    // token 16 tg + 4 g + r's 1 / D
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(O[0][r] * ir),
                                                       __float_as_uint(O[1][r] * ir), false, false);
      // streamed out: never re-read by this kernel
      __builtin_nontemporal_store(cvt_out<Tout>(__uint_as_float(sw[0])), orow + r * so_t);
      __builtin_nontemporal_store(cvt_out<Tout>(__uint_as_float(sw[1])), orow + (4 + r) * so_t);
    }
    if (den_out && ch == 0 && lane < 16)
      den_out[((long long)b * pr.T + tok0 + t) * pr.H + h] = D;
    orow += C * so_t;

    if (c + 1 < nc) {
      store32(st, tl, true, tid);
      flag_v(st);
      publish();
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_chunk_state32(const DevProblem& pr, int L, int n_seg, int n_used, int sp,
                                const void* k, const void* v, float* states, hipStream_t st) {
  if (pr.p != P || pr.dv != DV || pr.C != C) return hipErrorInvalidValue;
  if (sp < 0 || sp > L) return hipErrorInvalidValue;    // a spread range crosses one boundary
  const size_t lds = 2 * sizeof(StateTiles32);
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&chunk_state32_kernel), (int)lds);
  if (e != hipSuccess) return e;
  const SegGrid sg = make_seg_grid(pr, n_seg);
  if (sg.blocks() > 0x7fffffffLL) return hipErrorInvalidValue;
  launch_kernel(chunk_state32_kernel, dim3((unsigned)sg.blocks()), kThreads, lds, st,
      pr, sg, L, n_seg, n_used, sp, (const __bf16*)k, (const __bf16*)v, states);
  return hipGetLastError();
}

hipError_t launch_chunk_output32(const DevProblem& pr, bool out_bf16, int L, int n_seg, int sp,
                                 const void* q, const void* k, const void* v, void* o,
                                 float* den, const float* states, bool sum_prefix, hipStream_t st) {
  if (pr.p != P || pr.dv != DV || pr.C != C) return hipErrorInvalidValue;
  if (sp < 0 || sp > L || (sp > 0 && !sum_prefix)) return hipErrorInvalidValue;
  const size_t lds = sizeof(Walk32Lds);
  const SegGrid sg = make_seg_grid(pr, n_seg);
  if (sg.blocks() > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)sg.blocks());
  const __bf16 *qq = (const __bf16*)q, *kk = (const __bf16*)k, *vv = (const __bf16*)v;
  hipError_t e;
  if (out_bf16) {
    e = ensure_dynamic_lds(reinterpret_cast<const void*>(&chunk_output32_kernel<__bf16>), (int)lds);
    if (e != hipSuccess) return e;
    launch_kernel(chunk_output32_kernel<__bf16>, grid, kThreads, lds, st, pr, sg, L, n_seg, sp,
                  qq, kk, vv, (__bf16*)o, den, states, (int)sum_prefix);
  } else {
    e = ensure_dynamic_lds(reinterpret_cast<const void*>(&chunk_output32_kernel<float>), (int)lds);
    if (e != hipSuccess) return e;
    launch_kernel(chunk_output32_kernel<float>, grid, kThreads, lds, st, pr, sg, L, n_seg, sp,
                  qq, kk, vv, (float*)o, den, states, (int)sum_prefix);
  }
  return hipGetLastError();
}

}  // namespace kata

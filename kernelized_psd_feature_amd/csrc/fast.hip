// bf16 MFMA kernels for gfx950 (p = 16, d_v = 64, chunk C = 64): the chunk-state build and the
// segment walk of the chunked forward (intra-chunk tile + inter-chunk readout + output gate +
// state update), including KATA-Mg group widths 8 and 4.  (The quadratic form is in
// quadratic.hip.)
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
// inter-chunk denominator q^T Z q keeps fp32 accuracy: Z q runs on MFMA with Z split into a
// bf16 high part and a bf16 remainder (q is exact in bf16), the final dot with q in fp32.
//
#include <type_traits>

#include "device.h"
#include "kata.h"
#include "mfma_util.h"

namespace kata {
namespace {

constexpr int P = 16, DV = 64, C = 64, F = P * P;
constexpr int kThreads = 256;
constexpr int kStateFloats = F * (DV + 1);     // 16640: S (4 waves x 16 tiles x 256) + Z (256)
// LDS row strides (32 banks of 4 bytes; 4-, 8- and 16-byte accesses served 32, 16 and 8
// lanes at a time).  The q / k row reads, the transposed v reads and the K^T factor reads of
// one lane group avoid bank conflicts with these strides (the K^T rows with the placement
// below); the state's publish, 8-byte words at a 16-byte stride, does not.
constexpr int QROW = 20;                       // bf16 per q / k row: 40 B, 8-byte aligned
constexpr int KTROW = 68;                      // fp32 per row of the K^T tile
constexpr int VROW = 80;                       // bf16 per v row: 160 B, 16-byte aligned

// ---- chunk tiles in LDS ------------------------------------------------------------------
// kPacked adds rows to the K^T tile: 2 k (the weight of an off-diagonal packed state row) at
// rows KT_D + i and zeros (the padding rows of the packed layout) at rows KT_Z0 and KT_Z0 + 1.
// With the row stride KTROW = 68 a row's 16-byte reads start on bank group 4 (row mod 8); the
// rows one 8-lane group of the update reads hold k_i, 2 k_i, k_{i+2}, 2 k_{i+2} and a zero row
// for one parity of i (i = a + (t & 1), a even): the doubled rows sit 4 groups over
// (KT_D = 20) and the zero row has the other parity (KT_Z0 + 1 - (i & 1)), so the group's
// distinct rows fall on distinct bank groups.
constexpr int KT_D = 20, KT_Z0 = 36, KT_PACKED_ROWS = 38;
static_assert(KT_D % 8 == 4 && KT_D >= P && KT_Z0 >= KT_D + P && KT_Z0 % 8 == 4 &&
              KT_PACKED_ROWS == KT_Z0 + 2, "K^T row placement");
template <bool kPacked>
struct __align__(16) TilesT {
  __bf16 Qs[C][QROW];                 // q rows (bf16), row-major
  __bf16 Ks[C][QROW];                 // k rows (bf16), row-major
  float KT[kPacked ? KT_PACKED_ROWS : P][KTROW];   // k transposed, fp32 (exact copies)
  __bf16 V[C][VROW];                  // v rows (bf16), row-major
};
using Tiles = TilesT<false>;

// One thread's share of a chunk's global loads, held in registers while the previous chunk
// is computed.  Waves 0-1 carry half a q row each, waves 2-3 half a k row (which row and half:
// qk_piece); every thread carries 16 bytes of two consecutive v rows.
struct Stage {
  uint4 qk;
  uint4 v0, v1;
};

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

// The q or k row of the chunk and the 16-byte half of it that thread tid stages.  With q (the
// walk), lanes 2i and 2i+1 take the two halves of row 32 (w & 1) + i, so one load touches 32
// rows whole (in (B,T,H,D) order every 32-byte row sits in its own cache line) rather than half
// of each of 64 rows.  Without q (the state pass: k on waves 2-3) each lane takes one row and
// the wave picks the half, which measured faster there.
struct QkPiece {
  int row, half;
};
__device__ __forceinline__ QkPiece qk_piece(int tid, bool with_q) {
  return with_q ? QkPiece{32 * ((tid >> 6) & 1) + ((tid & 63) >> 1), tid & 1}
                : QkPiece{tid & 63, (tid >> 6) & 1};
}

__device__ __forceinline__ StagePtrs stage_ptrs(const DevProblem& pr, const __bf16* q,
                                                const __bf16* k, const __bf16* v, int b, int h,
                                                int tok0, bool with_q, int tid, int dir = 1) {
  StagePtrs sp;
  const int w = tid >> 6;
  const QkPiece pc = qk_piece(tid, with_q);        // q on waves 0-1, k on waves 2-3
  const int row = pc.row, half = pc.half;
  if (w < 2)
    sp.qk = with_q ? q + row_off(pr.sq, b, tok0 + row, h) + 8 * half : nullptr;
  else
    sp.qk = k + row_off(pr.sk, b, tok0 + row, h) + 8 * half;
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

template <bool kPacked>
__device__ __forceinline__ void stage_store(const Stage& st, TilesT<kPacked>& tl, bool with_q,
                                            int tid) {
  const int w = tid >> 6;
  const QkPiece pc = qk_piece(tid, with_q);
  const int row = pc.row, half = pc.half;
  if (w < 2) {
    if (with_q) {
      *reinterpret_cast<uint2*>(&tl.Qs[row][8 * half]) = uint2{st.qk.x, st.qk.y};
      *reinterpret_cast<uint2*>(&tl.Qs[row][8 * half + 4]) = uint2{st.qk.z, st.qk.w};
    }
  } else {
    if (with_q) {   // the row-major K tile feeds only the walk's score tiles
      *reinterpret_cast<uint2*>(&tl.Ks[row][8 * half]) = uint2{st.qk.x, st.qk.y};
      *reinterpret_cast<uint2*>(&tl.Ks[row][8 * half + 4]) = uint2{st.qk.z, st.qk.w};
    }
    const uint32_t wd[4] = {st.qk.x, st.qk.y, st.qk.z, st.qk.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf_lo(wd[e]), hi = bf_hi(wd[e]);
      tl.KT[8 * half + 2 * e][row] = lo;
      tl.KT[8 * half + 2 * e + 1][row] = hi;
      if (kPacked) {
        tl.KT[KT_D + 8 * half + 2 * e][row] = 2.f * lo;    // exact
        tl.KT[KT_D + 8 * half + 2 * e + 1][row] = 2.f * hi;
      }
    }
  }
  const int a = tid >> 3, c8 = tid & 7;
  *reinterpret_cast<uint4*>(&tl.V[2 * a][8 * c8]) = st.v0;
  *reinterpret_cast<uint4*>(&tl.V[2 * a + 1][8 * c8]) = st.v1;
}

// A operand of the state update for feature rows f = 16 i + (lane%16), i fixed, 32-key step
// m: phi_f(k_s) = k_s[i] k_s[j], slot order kappa.
template <class TL>
__device__ __forceinline__ bf16x8 phik_frag(const TL& tl, int i, int m, int lane) {
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

// Packed layout: tile t row 4g + r holds the state row of the pair (a + (t & 1), 4J + r),
// (a, J) the double group 4 (t >> 1) + g of the layout's list.

// A operand of the packed state update: row (lane % 16) of the tile is the pair (i, j);
// irow selects the K^T row for the i factor (i, KT_D + i for the doubled copy, a zero row).
template <class TL>
__device__ __forceinline__ bf16x8 phik_packed_frag(const TL& tl, int irow, int jrow, int m,
                                                   int lane) {
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

// k_s[i] for i = lane%16 over the slots of 32-key step m (A and B operand of Z = K^T K).
template <class TL>
__device__ __forceinline__ bf16x8 kcol_frag(const TL& tl, int m, int lane) {
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

// Squared-score tile of keys [s0, s0 + 16) (rows) against this lane's query t (column), from
// the A operand kf (k rows) and the B operand qf (q_t[4g .. 4g + 3]): the bf16 weights P of
// slots r = 0, 1 and 2, 3 as packed pairs pw, and their sum added to lsum (a bf16 pair dot with
// ones, so the sum is taken over the rounded weights).  kMask (the diagonal tile, keys
// 16w + 4g + r against token 16w + l16): the future keys' weights are +0.  GW < 16 (KATA-Mg, groups of GW
// coordinates): one product per group, the query operand cut to the lane groups holding that
// group's coordinates, and the squared group dots summed.
template <int GW, bool kMask>
__device__ __forceinline__ void score_tile(const s16x4& kf, const s16x4& qf, int lane,
                                           uint32_t (&pw)[2], float& lsum) {
  f32x4 x2;
  if constexpr (GW == P) {
    const f32x4 sc = mfma16(kf, qf, zero4());
#pragma unroll
    for (int r = 0; r < 4; ++r) x2[r] = sc[r] * sc[r];
  } else {
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
    // keys 16w + 4g + r against token 16w + l16: future for 4g + r > l16 (select, never
    // multiply: the lane masks are loop constants)
    const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) x2[r] = 4 * g + r <= l16 ? x2[r] : 0.f;
  }
  pw[0] = pack_bf16x2(x2[0], x2[1]);
  pw[1] = pack_bf16x2(x2[2], x2[3]);
  lsum = sum_bf16x2(pw[0], lsum);
  lsum = sum_bf16x2(pw[1], lsum);
}

// ==========================================================================================
// Per-layout constants shared by the state and walk kernels.
//   direct: 16 state tiles (tile = i, rows j), wave w owns tiles 4w .. 4w+3, 8 readout K steps.
//   packed: the double groups of the unique pairs (see mfma_util.h), two per 16-row tile:
//           10 tiles at GW = 16, 5 readout K steps.  Wave w owns tiles w, w + 4, w + 8, so
//           waves 0-1 own 3 and waves 2-3 (more intra-chunk work) own 2.
//   KATA-Mg (packed, groups of GW = 8 or 4 consecutive coordinates): only the double groups
//           inside one group exist, 6 or 4 tiles.
// Fragment layout of a state (floats): tile t, value tile nt, lane -> ((t*4 + nt)*64 +
// lane)*4 .. +3 (the accumulator registers as they are), then Z as one 16 x 16 tile; the
// workspace holds it as it is or, for packed states through the scan, without the zero rows
// (Stored, below).
// ==========================================================================================
template <bool kPacked, int GW = P>
struct Layout {
  static_assert(kPacked || GW == P, "the direct layout is ungrouped");
  static_assert(GW == 16 || GW == 8 || GW == 4, "group width");
  static constexpr int kGroupDG = (GW / 4) * (GW / 4 + 1);   // double groups in one group
  static constexpr int kTiles = kPacked ? (P / GW) * kGroupDG / 2 : 16;
  static constexpr int kSlots = (kTiles + 3) / 4;        // state tiles a wave can own
  static constexpr int kSteps = kTiles / 2;              // readout K steps of 32 rows
  static constexpr int kZOff = kTiles * 16 * DV;         // offset of Z in a stored state
  static constexpr int kStateFloats = kZOff + 256;
  __device__ static bool owns(int w, int slot) { return !kPacked || w + 4 * slot < kTiles; }
  __device__ static int tile(int w, int slot) { return kPacked ? w + 4 * slot : 4 * w + slot; }
  // double group idx of the (grouped) list -> (a, J)
  __device__ static void dg(int idx, int& a, int& J) {
    const int grp = idx / kGroupDG;
    double_group(idx - grp * kGroupDG, a, J);
    a += grp * GW;
    J += grp * (GW / 4);
  }
};
static_assert(Layout<false>::kStateFloats == kStateFloats, "direct state size");
static_assert(Layout<true>::kTiles == 10 && Layout<true, 8>::kTiles == 6 &&
              Layout<true, 4>::kTiles == 4, "packed tile counts (plan.cpp)");

// A state as stored in the workspace (state pass -> scan -> walk).  The direct layout, and the
// packed ones when the walks add the segment states themselves (few segments), store the
// fragments as they are (above).  With the segment scan (DevProblem::stored_compact), the
// packed states leave out their zero rows.  A packed fragment (tile t, lane group gp) holds rows
// j = 4 J + r, r = 0..3, of double group (a, J) = Layout::dg(4 (t / 2) + gp) at i = a + t % 2;
// its rows with i > j (inside the diagonal double groups) are zero in every state and are
// not stored: blocks [t][nt][gp] of 16 columns c x (stored rows), column-major, so a lane's
// rows sit together (one 16-byte access for a whole fragment), then Z as one 16 x 16 tile
// (lane-major).  That leaves the p (GW + 1) / 2 unique pairs' rows: 136 of the 160 rows at
// GW = 16, 15 % fewer bytes for each state the step writes, scans and reads.
template <int GW>
struct StoredPacked {
  static constexpr int kTiles = Layout<true, GW>::kTiles;
  unsigned char mask[kTiles][4];      // bit r: row r of fragment (t, gp) is stored
  int base[kTiles][4];                // float offset of block (t, nt = 0, gp)
  int stride[kTiles];                 // floats from value tile nt to nt + 1 of tile t
  int zoff;                           // float offset of Z
};
constexpr int dg_J(int idx) {
  int J = 0;
  while ((J + 1) * (J + 2) <= idx) ++J;
  return J;
}
template <int GW>
constexpr StoredPacked<GW> make_stored_packed() {
  using LY = Layout<true, GW>;
  StoredPacked<GW> sp{};
  int off = 0;
  for (int t = 0; t < LY::kTiles; ++t) {
    int rows = 0;
    for (int gp = 0; gp < 4; ++gp) {
      const int idx = 4 * (t >> 1) + gp, grp = idx / LY::kGroupDG, loc = idx - grp * LY::kGroupDG;
      const int J0 = dg_J(loc), a = 2 * (loc - J0 * (J0 + 1)) + grp * GW;
      const int J = J0 + grp * (GW / 4), i = a + (t & 1);
      int m = 0, n = 0;
      for (int r = 0; r < 4; ++r)
        if (i <= 4 * J + r) { m |= 1 << r; ++n; }
      sp.mask[t][gp] = (unsigned char)m;
      sp.base[t][gp] = off + 16 * rows;
      rows += n;
    }
    sp.stride[t] = 16 * rows;
    off += 4 * 16 * rows;
  }
  sp.zoff = off;
  return sp;
}
template <bool kPacked, int GW>
struct Stored {
  static constexpr int kZOffFull = Layout<kPacked, GW>::kZOff;
  static constexpr int kZOffCompact = kPacked ? make_stored_packed<GW>().zoff : kZOffFull;
  __device__ static int zoff(bool compact) { return compact ? kZOffCompact : kZOffFull; }
  __device__ static int floats(bool compact) { return zoff(compact) + 256; }
};
// the unique pairs of each group, the count the planner sizes the workspace with (plan.cpp)
static_assert(Stored<true, 16>::kZOffCompact == 16 * 17 / 2 * DV &&
              Stored<true, 8>::kZOffCompact == 16 * 9 / 2 * DV &&
              Stored<true, 4>::kZOffCompact == 16 * 5 / 2 * DV &&
              Stored<false, P>::kZOffFull + 256 == kStateFloats, "stored state sizes");
__constant__ StoredPacked<16> kStored16 = make_stored_packed<16>();
__constant__ StoredPacked<8> kStored8 = make_stored_packed<8>();
__constant__ StoredPacked<4> kStored4 = make_stored_packed<4>();
template <int GW>
__device__ __forceinline__ const StoredPacked<GW>& stored_packed() {
  if constexpr (GW == 16) return kStored16;
  else if constexpr (GW == 8) return kStored8;
  else return kStored4;
}

// Where one lane's fragment of tile t (rows 4 (slot / 16) + r, column 16 nt + slot % 16)
// sits in a stored state: float offset off + nt * stride, its stored rows (bit r of mask) in
// order.  The stored rows of a fragment are always its top ones (masks 0xF, 0xE, 0xC, 0x8:
// i > j holds for the first rows j = 4 J + r), so row r of a fragment with n stored rows is
// float r - (4 - n) from off.  slot is the lane of the fragment's owner in the state's layout.
template <bool kPacked, int GW, bool kCompact>
struct FragPlace {
  static constexpr bool compact = kPacked && kCompact;
  int off, stride, mask;
  __device__ __forceinline__ void init(int t, int slot) {
    if constexpr (!compact) {
      off = (t * 4 * 64 + slot) * 4;
      stride = 64 * 4;
      mask = 0xF;
    } else {
      const StoredPacked<GW>& sp = stored_packed<GW>();
      const int gp = slot >> 4;
      mask = sp.mask[t][gp];
      off = sp.base[t][gp] + (slot & 15) * __builtin_popcount(mask);
      stride = sp.stride[t];
    }
  }
  __device__ __forceinline__ void store(float* out, int nt, const f32x4& x) const {
    float* o = out + off + nt * stride;
    if (!compact || mask == 0xF) {     // constant, or one lane group's mask
      *reinterpret_cast<f32x4*>(o) = x;
    } else {
#pragma unroll
      for (int r = 1; r < 4; ++r)          // bit 0 is set only in whole fragments
        if ((mask >> r) & 1) o[__builtin_popcount(mask & ((1 << r) - 1))] = x[r];
    }
  }
  // Branch-free, so the loads of all fragments are in flight together: the four floats from
  // row 0's place (before off when rows are missing: the previous lane's or block's floats,
  // inside the state since the state's first fragment is whole), the missing rows' values
  // replaced by zero.
  __device__ __forceinline__ void add(const float* in, int nt, f32x4& x) const {
    if constexpr (!compact) {
      x += *reinterpret_cast<const f32x4*>(in + off + nt * stride);
    } else {
      const int miss = 4 - __builtin_popcount(mask);
      const float* q = in + off + nt * stride - miss;
      float v[4];
      __builtin_memcpy(v, q, sizeof(v));
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] += r >= miss ? v[r] : 0.f;
    }
  }
};
// f(std::true_type) for compactly stored states, f(std::false_type) otherwise: the layout is
// a compile-time choice inside f, and the one branch on the wave-uniform flag sits outside it
template <class F>
__device__ __forceinline__ void with_stored_layout(bool compact, F&& f) {
  if (compact) f(std::true_type{});
  else f(std::false_type{});
}

// Row sources of the packed update's A operand for this lane's row of each owned tile.
template <bool kPacked, int GW>
struct UpdateRows {
  using LY = Layout<kPacked, GW>;
  int irow[LY::kSlots], jrow[LY::kSlots];
  __device__ void init(int w, int lane) {
#pragma unroll
    for (int sl = 0; sl < LY::kSlots; ++sl) {
      if (!kPacked) {
        irow[sl] = 4 * w + sl;                  // broadcast row i of the tile
        jrow[sl] = lane & 15;
      } else {
        const int t = LY::owns(w, sl) ? LY::tile(w, sl) : 0, row = lane & 15;
        int a, J;
        LY::dg(4 * (t >> 1) + (row >> 2), a, J);
        const int i = a + (t & 1), j = 4 * J + (row & 3);
        irow[sl] = i > j ? KT_Z0 + 1 - (i & 1) : (i == j ? i : KT_D + i);
        jrow[sl] = j;
      }
    }
  }
};

// S[slot] += Phi(K)^T V over one staged chunk, and Z += K^T K if with_z.
template <bool kPacked, int GW, class TL>
__device__ __forceinline__ void state_update(const TL& tl, const UpdateRows<kPacked, GW>& ur,
                                             f32x4 (&S)[Layout<kPacked, GW>::kSlots][4],
                                             f32x4& Z, int w, int lane, bool with_z) {
  using LY = Layout<kPacked, GW>;
  // both 32-key steps unrolled: the LDS addresses of the second become immediate offsets
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    bf16x8 vb[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) vb[nt] = v_frag(tl.V, m, nt, lane);
#pragma unroll
    for (int sl = 0; sl < LY::kSlots; ++sl) {
      if (!LY::owns(w, sl)) continue;
      const bf16x8 a = kPacked ? phik_packed_frag(tl, ur.irow[sl], ur.jrow[sl], m, lane)
                               : phik_frag(tl, ur.irow[sl], m, lane);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[sl][nt] = mfma32(a, vb[nt], S[sl][nt]);
    }
    if (with_z) {
      const bf16x8 kf = kcol_frag(tl, m, lane);
      Z = mfma32(kf, kf, Z);
    }
  }
}

// One 32-key step m of the S update from value fragments vb the caller already holds (the walk
// shares them with its P.V step).
template <bool kPacked, int GW, class TL>
__device__ __forceinline__ void state_update_step(const TL& tl, const UpdateRows<kPacked, GW>& ur,
                                                  f32x4 (&S)[Layout<kPacked, GW>::kSlots][4],
                                                  const bf16x8 (&vb)[4], int w, int m,
                                                  int lane) {
  using LY = Layout<kPacked, GW>;
#pragma unroll
  for (int sl = 0; sl < LY::kSlots; ++sl) {
    if (!LY::owns(w, sl)) continue;
    const bf16x8 a = kPacked ? phik_packed_frag(tl, ur.irow[sl], ur.jrow[sl], m, lane)
                             : phik_frag(tl, ur.irow[sl], m, lane);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[sl][nt] = mfma32(a, vb[nt], S[sl][nt]);
  }
}

template <bool kPacked>
__device__ __forceinline__ void zero_pad_rows(TilesT<kPacked>& tl, int tid) {
  if (kPacked && tid < 2 * KTROW) tl.KT[kPacked ? KT_Z0 + tid / KTROW : 0][tid % KTROW] = 0.f;
}

// ==========================================================================================
// Segment state: S_seg = sum over the segment's chunks of Phi(K_c)^T V_c and Z_seg = sum K^T K.
// One workgroup per (segment, head, batch), XCD-aware (SegGrid).
// ==========================================================================================
template <bool kPacked, int GW>
__global__ __launch_bounds__(kThreads, 3) void chunk_state_fast_kernel(
    DevProblem pr, SegGrid sg, int L, int n_seg, int n_used, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, float* __restrict__ states) {
  using LY = Layout<kPacked, GW>;
  __shared__ TilesT<kPacked> tl[2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const SegBlock blk = seg_block(sg, pr.H);
  if (!blk.live) return;                           // padding of the grid (whole workgroup)
  const int seg = blk.seg, h = blk.h, b = blk.b;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);
  const long long sv_t = pr.sv[1];
  const int n_stored = Stored<kPacked, GW>::floats(pr.stored_compact);
  if (seg >= n_used) {
    // a state no prefix needs (the last segment's, in the forward): zeros for the scan, and
    // its k, v are not read
    float4* out = reinterpret_cast<float4*>(
        states + ((long long)(b * pr.H + h) * n_seg + seg) * n_stored);
    for (int x = tid; x < n_stored / 4; x += kThreads) out[x] = float4{0.f, 0.f, 0.f, 0.f};
    return;
  }

  f32x4 S[LY::kSlots][4];
#pragma unroll
  for (int sl = 0; sl < LY::kSlots; ++sl)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[sl][nt] = zero4();
  f32x4 Z = zero4();
  UpdateRows<kPacked, GW> ur;
  ur.init(w, lane);
  zero_pad_rows(tl[0], tid);
  zero_pad_rows(tl[1], tid);

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
  auto step = [&](int c, Stage& next) {
    state_update<kPacked, GW>(tl[c & 1], ur, S, Z, w, lane, w == 0);
    // the other buffer was last read in the previous iteration, before its barrier
    if (c + 1 < nc) stage_store(next, tl[(c + 1) & 1], false, tid);
    if (c + 3 < nc) { sp.next(); stage_load(next, sp, sv_t); }   // chunk c + 3
    __syncthreads();
  };
  for (int c = 0; c < nc; c += 2) {
    step(c, sa);                     // chunk c+1 is in sa, chunk c+2 in sb
    if (c + 1 < nc) step(c + 1, sb);
  }
  float* out = states + ((long long)(b * pr.H + h) * n_seg + seg) * n_stored;
  with_stored_layout(pr.stored_compact, [&](auto compact) {
#pragma unroll
    for (int sl = 0; sl < LY::kSlots; ++sl) {
      if (!LY::owns(w, sl)) continue;
      FragPlace<kPacked, GW, decltype(compact)::value> fp;
      fp.init(LY::tile(w, sl), lane);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) fp.store(out, nt, S[sl][nt]);
    }
  });
  if (w == 0)
    *reinterpret_cast<f32x4*>(out + Stored<kPacked, GW>::zoff(pr.stored_compact) + lane * 4) = Z;
}

// ==========================================================================================
// Segment state, single feature group: the same sums as chunk_state_fast_kernel with phi(k)
// formed from lane broadcasts instead of LDS re-reads.  The chunk's k rows sit row-major in
// LDS; one transposed read per 32-key step hands lane (g, j) the value k_s[j] (j = lane % 16)
// of the 8 keys s of its MFMA slots, and the keys of a lane group g are the same for all 16
// lanes of its row.  Row i of direct state tile i then needs k_s[i] from lane i of the same
// row: a DPP row broadcast folded into the multiply (v_mul_f32 with row_newbcast:i).  Each
// wave owns direct tiles 4w .. 4w+3 (rows (i, j) for every j) and the same transposed read
// is the A and B operand of Z = K^T K.  Per chunk and workgroup this moves about 50 KB
// through LDS instead of 132 KB (the fp32 K^T rows read for every phi product).
// Outputs: the direct layout as it is, or the packed one by a lane remap (see
// store_packed_from_direct).  The products and their summation order are those of
// chunk_state_fast_kernel, so the states are the same bit for bit (zero rows: +0).
// ==========================================================================================
constexpr int KSROW = 24;                     // bf16 per k row: 48 B, 16-byte aligned rows

struct __align__(16) KvTiles {
  __bf16 K[C][KSROW];                 // k rows (bf16), row-major
  __bf16 V[C][VROW];                  // v rows (bf16), row-major
};

template <int I>
__device__ __forceinline__ float row_bcast(float x) {   // lane I of each 16-lane row
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + I, 0xF, 0xF, true));
}

// A operand of direct tile I for one 32-key step: slot r = k_s[I] k_s[j], from this lane's
// k_s[j] values kf (fp32 copies of bf16, so every product is exact before its bf16 rounding)
template <int I>
__device__ __forceinline__ bf16x8 phik_bcast(const float (&kf)[8]) {
  bf16x8 f;
#pragma unroll
  for (int r = 0; r < 8; ++r) f[r] = (__bf16)(row_bcast<I>(kf[r]) * kf[r]);
  return f;
}

// Direct tile i's accumulators (lane (g, c): rows j = 4g + r, column 16 nt + c) written into
// the packed layout: the pair (i, j) lives in double group (a, J) = (i - i % 2, g) of column
// block J = g, i.e. packed tile 2 (idx / 4) + i % 2, lane group idx % 4, idx = J (J + 1) + a / 2,
// same register r; off-diagonal rows carry weight 2 (exact), pairs with i > j inside a double
// group are zero rows, and lane groups with i > 4g + 3 hold no packed row.
template <bool kCompact>
__device__ __forceinline__ void store_packed_from_direct(float* out, int i, const f32x4 (&S)[4],
                                                        int lane) {
  const int g = lane >> 4, c = lane & 15;
  if (i > 4 * g + 3) return;
  const int idx = g * (g + 1) + (i >> 1);
  const int t = 2 * (idx >> 2) + (i & 1), gp = idx & 3;
  FragPlace<true, P, kCompact> fp;
  fp.init(t, 16 * gp + c);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * g + r;
      x[r] = i < j ? 2.f * S[nt][r] : (i == j ? S[nt][r] : 0.f);
    }
    fp.store(out, nt, x);
  }
}

struct StageKv {
  uint4 k;         // waves 2-3: 16 bytes of a k row
  uint4 v0, v1;    // 16 bytes of two consecutive v rows
};

// The state sum of wave W's four direct tiles over the segment's chunks (the loop of
// chunk_state_dpp_kernel, one instance per wave so that the broadcast lanes are constants).
template <int W>
__device__ __forceinline__ void state_dpp_loop(KvTiles (&tl)[2], const __bf16* kp, const __bf16* vp,
                                               long long k_step, long long v_step, long long sv_t,
                                               int nc, int tid, f32x4 (&S)[4][4], f32x4& Z) {
  const int lane = tid & 63;
  const int krow = tid & 63, khalf = (tid >> 6) & 1, a = tid >> 3, c8 = tid & 7;
  auto load = [&](StageKv& x) {
    if (W >= 2) x.k = ld16(kp);
    x.v0 = ld16(vp);
    x.v1 = ld16(vp + sv_t);
  };
  auto store = [&](const StageKv& x, KvTiles& t) {
    if (W >= 2) *reinterpret_cast<uint4*>(&t.K[krow][8 * khalf]) = x.k;
    *reinterpret_cast<uint4*>(&t.V[2 * a][8 * c8]) = x.v0;
    *reinterpret_cast<uint4*>(&t.V[2 * a + 1][8 * c8]) = x.v1;
  };
  auto advance = [&]() {
    kp += k_step;
    vp += v_step;
  };
  StageKv sa, sb;
  load(sa);
  store(sa, tl[0]);
  if (nc > 1) { advance(); load(sa); }
  if (nc > 2) { advance(); load(sb); }
  __syncthreads();
  auto step = [&](int c, StageKv& next) {
    const KvTiles& t = tl[c & 1];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bf16x8 kt = v_frag(t.K, m, 0, lane);      // k_s[lane % 16] of this lane's keys
      float kf[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) kf[r] = (float)kt[r];
      bf16x8 vb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) vb[nt] = v_frag(t.V, m, nt, lane);
      const bf16x8 a0 = phik_bcast<4 * W>(kf), a1 = phik_bcast<4 * W + 1>(kf);
      const bf16x8 a2 = phik_bcast<4 * W + 2>(kf), a3 = phik_bcast<4 * W + 3>(kf);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        S[0][nt] = mfma32(a0, vb[nt], S[0][nt]);
        S[1][nt] = mfma32(a1, vb[nt], S[1][nt]);
        S[2][nt] = mfma32(a2, vb[nt], S[2][nt]);
        S[3][nt] = mfma32(a3, vb[nt], S[3][nt]);
      }
      if (W == 0) Z = mfma32(kt, kt, Z);
    }
    // the other buffer was last read in the previous iteration, before its barrier
    if (c + 1 < nc) store(next, tl[(c + 1) & 1]);
    if (c + 3 < nc) { advance(); load(next); }         // chunk c + 3
    __syncthreads();
  };
  for (int c = 0; c < nc; c += 2) {
    step(c, sa);                       // chunk c+1 is in sa, chunk c+2 in sb
    if (c + 1 < nc) step(c + 1, sb);
  }
}

template <bool kPackedOut>
__global__ __launch_bounds__(kThreads, 3) void chunk_state_dpp_kernel(
    DevProblem pr, SegGrid sg, int L, int n_seg, int n_used, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, float* __restrict__ states) {
  using LY = Layout<kPackedOut, P>;
  __shared__ KvTiles tl[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SegBlock blk = seg_block(sg, pr.H);
  if (!blk.live) return;                           // padding of the grid (whole workgroup)
  const int seg = blk.seg, h = blk.h, b = blk.b;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);
  using ST = Stored<kPackedOut, P>;
  float* out = states + ((long long)(b * pr.H + h) * n_seg + seg) * ST::floats(pr.stored_compact);
  if (seg >= n_used) {
    // a state no prefix needs (the last segment's, in the forward): zeros, k and v unread
    for (int x = tid; x < ST::floats(pr.stored_compact) / 4; x += kThreads)
      reinterpret_cast<float4*>(out)[x] = float4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  f32x4 S[4][4];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[sl][nt] = zero4();
  f32x4 Z = zero4();
  // the segment is read last chunk first (the sum is order-free; the walk that follows starts
  // on the segment's first chunks, then the most recently read)
  const int tok_last = (c0 + nc - 1) * C;
  const __bf16* kp = k + row_off(pr.sk, b, tok_last + (tid & 63), h) + 8 * ((tid >> 6) & 1);
  const __bf16* vp = v + row_off(pr.sv, b, tok_last + 2 * (tid >> 3), h) + 8 * (tid & 7);
  const long long k_step = -(long long)C * pr.sk[1], v_step = -(long long)C * pr.sv[1];
  switch (w) {
    case 0: state_dpp_loop<0>(tl, kp, vp, k_step, v_step, pr.sv[1], nc, tid, S, Z); break;
    case 1: state_dpp_loop<1>(tl, kp, vp, k_step, v_step, pr.sv[1], nc, tid, S, Z); break;
    case 2: state_dpp_loop<2>(tl, kp, vp, k_step, v_step, pr.sv[1], nc, tid, S, Z); break;
    default: state_dpp_loop<3>(tl, kp, vp, k_step, v_step, pr.sv[1], nc, tid, S, Z); break;
  }
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    const int i = 4 * w + sl;
    if (kPackedOut) {
      with_stored_layout(pr.stored_compact, [&](auto compact) {
        store_packed_from_direct<decltype(compact)::value>(out, i, S[sl], lane);
      });
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        *reinterpret_cast<f32x4*>(out + ((i * 4 + nt) * 64 + lane) * 4) = S[sl][nt];
    }
  }
  if (w == 0) *reinterpret_cast<f32x4*>(out + ST::zoff(pr.stored_compact) + lane * 4) = Z;
}

// ==========================================================================================
// Segment state, single feature group, packed output: the packed state needs the 136 pairs
// i <= j only, so instead of 16 direct tiles the kernel runs 11:
//   broadcast tiles  direct tiles i = 0 .. 7 formed as in chunk_state_dpp_kernel (rows (i, j)
//                    for every j; their packed rows are those with j >= i),
//   gathered tiles   three tiles of the pairs (i, j) with 8 <= i <= j, formed from fp32 copies
//                    of k coordinates 8 .. 15 in LDS as in chunk_state_fast_kernel.  They hold
//                    exactly the twelve packed row quads (i, J) = (i, 4J .. 4J + 3) with i >= 8
//                    (J = 2: i = 8 .. 11; J = 3: i = 8 .. 15), quad q in lane group q % 4 of
//                    tile q / 4, so each lane stores its four rows with one 16-byte write.
// Wave w owns broadcast tiles 2w, 2w + 1 and gathered tile w (w < 3); wave 3 also forms Z.
// Against 16 broadcast tiles: 88 instead of 128 MFMAs and ~30 % less VALU per chunk, for
// 24 KB more LDS reads; the same products summed in the same order, so the same states.
// ==========================================================================================
constexpr int KT8ROWS = 2 * 8 + 1;            // k_8..15, 2 k_8..15, zeros

struct __align__(16) KvktTiles {
  __bf16 K[C][KSROW];                 // k rows (bf16), row-major
  __bf16 V[C][VROW];                  // v rows (bf16), row-major
  float KT[KT8ROWS][KTROW];           // coordinates 8 .. 15 of k transposed, fp32 (exact)
};

// quad q = 0 .. 11 of the gathered tiles -> (i, J)
__device__ __forceinline__ void gathered_quad(int q, int& i, int& J) {
  J = q < 4 ? 2 : 3;
  i = q < 4 ? 8 + q : 8 + (q - 4);
}

template <int W>
__device__ __forceinline__ void state_hybrid_loop(KvktTiles (&tl)[2], const __bf16* kp,
                                                  const __bf16* vp, long long k_step,
                                                  long long v_step, long long sv_t, int nc,
                                                  int tid, f32x4 (&S)[3][4], f32x4& Z) {
  const int lane = tid & 63;
  const int krow = tid & 63, khalf = (tid >> 6) & 1, a = tid >> 3, c8 = tid & 7;
  // this lane's row of gathered tile W: pair (i, j) -> K^T rows (i for the diagonal, the
  // doubled copy above it, the zero row below it) and j
  int irow = 2 * 8, jrow = 0;
  if (W < 3) {
    int i, J;
    gathered_quad(4 * W + ((lane & 15) >> 2), i, J);
    const int j = 4 * J + (lane & 3);
    irow = i > j ? 2 * 8 : (i == j ? i - 8 : 8 + i - 8);
    jrow = j - 8;
  }
  auto load = [&](StageKv& x) {
    if (W >= 2) x.k = ld16(kp);
    x.v0 = ld16(vp);
    x.v1 = ld16(vp + sv_t);
  };
  auto store = [&](const StageKv& x, KvktTiles& t) {
    if (W >= 2) *reinterpret_cast<uint4*>(&t.K[krow][8 * khalf]) = x.k;
    if (W == 3) {                                  // coordinates 8 .. 15 of row krow
      const uint32_t wd[4] = {x.k.x, x.k.y, x.k.z, x.k.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf_lo(wd[e]), hi = bf_hi(wd[e]);
        t.KT[2 * e][krow] = lo;
        t.KT[2 * e + 1][krow] = hi;
        t.KT[8 + 2 * e][krow] = 2.f * lo;            // exact
        t.KT[8 + 2 * e + 1][krow] = 2.f * hi;
      }
    }
    *reinterpret_cast<uint4*>(&t.V[2 * a][8 * c8]) = x.v0;
    *reinterpret_cast<uint4*>(&t.V[2 * a + 1][8 * c8]) = x.v1;
  };
  auto advance = [&]() {
    kp += k_step;
    vp += v_step;
  };
  StageKv sa, sb;
  load(sa);
  store(sa, tl[0]);
  if (nc > 1) { advance(); load(sa); }
  if (nc > 2) { advance(); load(sb); }
  __syncthreads();
  auto step = [&](int c, StageKv& next) {
    const KvktTiles& t = tl[c & 1];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      // the A operands first, then one value tile at a time (fewer registers live at once)
      bf16x8 a2;
      if (W < 3) a2 = phik_packed_frag(t, irow, jrow, m, lane);
      const bf16x8 kt = v_frag(t.K, m, 0, lane);      // k_s[lane % 16] of this lane's keys
      float kf[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) kf[r] = (float)kt[r];
      const bf16x8 a0 = phik_bcast<2 * W>(kf), a1 = phik_bcast<2 * W + 1>(kf);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8 vb = v_frag(t.V, m, nt, lane);
        S[0][nt] = mfma32(a0, vb, S[0][nt]);
        S[1][nt] = mfma32(a1, vb, S[1][nt]);
        if (W < 3) S[2][nt] = mfma32(a2, vb, S[2][nt]);
      }
      if (W == 3) Z = mfma32(kt, kt, Z);
    }
    // the other buffer was last read in the previous iteration, before its barrier
    if (c + 1 < nc) store(next, tl[(c + 1) & 1]);
    if (c + 3 < nc) { advance(); load(next); }         // chunk c + 3
    __syncthreads();
  };
  for (int c = 0; c < nc; c += 2) {
    step(c, sa);                       // chunk c+1 is in sa, chunk c+2 in sb
    if (c + 1 < nc) step(c + 1, sb);
  }
}

__global__ __launch_bounds__(kThreads, 3) void chunk_state_hybrid_kernel(
    DevProblem pr, SegGrid sg, int L, int n_seg, int n_used, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, float* __restrict__ states) {
  using LY = Layout<true, P>;
  __shared__ KvktTiles tl[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SegBlock blk = seg_block(sg, pr.H);
  if (!blk.live) return;                           // padding of the grid (whole workgroup)
  const int seg = blk.seg, h = blk.h, b = blk.b;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);
  using ST = Stored<true, P>;
  float* out = states + ((long long)(b * pr.H + h) * n_seg + seg) * ST::floats(pr.stored_compact);
  if (seg >= n_used) {
    // a state no prefix needs (the last segment's, in the forward): zeros, k and v unread
    for (int x = tid; x < ST::floats(pr.stored_compact) / 4; x += kThreads)
      reinterpret_cast<float4*>(out)[x] = float4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  if (tid < KTROW) {                               // the zero row of both buffers
    tl[0].KT[2 * 8][tid] = 0.f;
    tl[1].KT[2 * 8][tid] = 0.f;
  }
  f32x4 S[3][4];
#pragma unroll
  for (int sl = 0; sl < 3; ++sl)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[sl][nt] = zero4();
  f32x4 Z = zero4();
  // the segment is read last chunk first (the sum is order-free; the walk that follows starts
  // on the segment's first chunks, then the most recently read)
  const int tok_last = (c0 + nc - 1) * C;
  const __bf16* kp = k + row_off(pr.sk, b, tok_last + (tid & 63), h) + 8 * ((tid >> 6) & 1);
  const __bf16* vp = v + row_off(pr.sv, b, tok_last + 2 * (tid >> 3), h) + 8 * (tid & 7);
  const long long k_step = -(long long)C * pr.sk[1], v_step = -(long long)C * pr.sv[1];
  switch (w) {
    case 0: state_hybrid_loop<0>(tl, kp, vp, k_step, v_step, pr.sv[1], nc, tid, S, Z); break;
    case 1: state_hybrid_loop<1>(tl, kp, vp, k_step, v_step, pr.sv[1], nc, tid, S, Z); break;
    case 2: state_hybrid_loop<2>(tl, kp, vp, k_step, v_step, pr.sv[1], nc, tid, S, Z); break;
    default: state_hybrid_loop<3>(tl, kp, vp, k_step, v_step, pr.sv[1], nc, tid, S, Z); break;
  }
  with_stored_layout(pr.stored_compact, [&](auto compact) {
    store_packed_from_direct<decltype(compact)::value>(out, 2 * w, S[0], lane);
    store_packed_from_direct<decltype(compact)::value>(out, 2 * w + 1, S[1], lane);
  });
  if (w < 3) {
    // gathered quad 4w + g of this lane: rows (i, 4J + r) -> packed tile 2 (idx / 4) + i % 2,
    // lane group idx % 4, idx = J (J + 1) + (i - i % 2) / 2, the same register r
    const int g = lane >> 4, c = lane & 15;
    int i, J;
    gathered_quad(4 * w + g, i, J);
    const int idx = J * (J + 1) + (i >> 1);
    const int t = 2 * (idx >> 2) + (i & 1), gp = idx & 3;
    with_stored_layout(pr.stored_compact, [&](auto compact) {
      FragPlace<true, P, decltype(compact)::value> fp;
      fp.init(t, 16 * gp + c);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) fp.store(out, nt, S[2][nt]);
    });
  } else {
    *reinterpret_cast<f32x4*>(out + ST::zoff(pr.stored_compact) + lane * 4) = Z;
  }
}

// ==========================================================================================
// Segment walk: start from the segment's exclusive prefix (S_{<c}, Z_{<c}); for every chunk,
// outputs = (readout of the prefix + causal intra-chunk tile) / (eps + denominators), then
// the chunk's own state is added.  One workgroup per (segment, head, batch) (SegGrid).
//   Each wave owns some state tiles (fp32, in registers, as in the state kernel) and the
//   chunk's tokens [16 w, 16 w + 16).  Once per chunk every wave publishes its state tiles in
//   LDS as bf16 MFMA operands; each wave then reads out its own tokens over all state rows, so no
//   partial outputs cross waves.
// ==========================================================================================
// Readout K order of the single-group packed walk: the double group (a, J), a = 2A, that lane
// group g reads out in K step kk.  Steps 0-3 take the 2 x 2 block (A, J) = (g % 2 + TA,
// g / 2 + TJ) at (TA, TJ) = (0, 0), (0, 2), (2, 1), (4, 2); step 4 takes (A, J) = (2, 3), (3, 3),
// (6, 3), (7, 3).  The five steps hold the 20 double groups once each, and in steps 0-3 a
// lane's q offsets move from step to step by constants only: the readout addresses q with 4
// registers instead of 10.
struct RoBlock {
  int A, J;
};
__host__ __device__ constexpr RoBlock ro_block(int kk, int g) {
  return kk == 0 ? RoBlock{g % 2, g / 2}
       : kk == 1 ? RoBlock{g % 2, g / 2 + 2}
       : kk == 2 ? RoBlock{g % 2 + 2, g / 2 + 1}
       : kk == 3 ? RoBlock{g % 2 + 4, g / 2 + 2}
                 : RoBlock{2 + g % 2 + 4 * (g / 2), 3};
}
// 4 kk + g of the step and lane group holding double group (2A, J)
__host__ __device__ constexpr int ro_slot(int A, int J) {
  for (int kk = 0; kk < 5; ++kk)
    for (int g = 0; g < 4; ++g)
      if (ro_block(kk, g).A == A && ro_block(kk, g).J == J) return 4 * kk + g;
  return -1;
}
constexpr bool ro_order_ok() {
  bool seen[8][4] = {};
  for (int kk = 0; kk < 5; ++kk)
    for (int g = 0; g < 4; ++g) {
      const RoBlock b = ro_block(kk, g);
      if (b.A < 0 || b.A > 7 || b.J < 0 || b.J > 3 || b.A > 2 * b.J + 1 || seen[b.A][b.J])
        return false;
      seen[b.A][b.J] = true;
    }
  return true;
}
static_assert(ro_order_ok() && Layout<true, P>::kSteps == 5, "readout K order: 20 double groups");

template <bool kPacked, int GW>
struct __align__(16) WalkLds {
  TilesT<kPacked> tl;
  uint4 Sb[Layout<kPacked, GW>::kSteps][4][64];   // S_{<c} as MFMA operands: [K step][value tile][lane]
  uint4 Zb[kPacked ? 64 : 1];                 // Z_{<c} as bf16 hi / lo A operands (packed layouts)
  float den[C];                               // D_t of the chunk's tokens
  float inv[C];                               // 1 / D_t
  uint32_t vbad[4];                           // per wave: its staged v rows hold a non-finite value
};

static_assert(sizeof(WalkLds<false, P>) <= 160 * 1024 / 3 && sizeof(WalkLds<true, P>) <= 160 * 1024 / 3,
              "three walks per CU");

// kCompact: the segment states are stored without their zero rows (pr.stored_compact); a
// template parameter, so that each walk holds one form of the prefix load
template <typename Tout, bool kPacked, int GW, bool kCompact>
__global__ __launch_bounds__(kThreads, 3) void chunk_output_fast_kernel(
    DevProblem pr, SegGrid sg, int L, int n_seg, const __bf16* __restrict__ q,
    const __bf16* __restrict__ k, const __bf16* __restrict__ v, Tout* __restrict__ o,
    float* __restrict__ den_out, const float* __restrict__ states, int sum_prefix) {
  using LY = Layout<kPacked, GW>;
  __shared__ WalkLds<kPacked, GW> sm;
  TilesT<kPacked>& tl = sm.tl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const SegBlock blk = seg_block(sg, pr.H);
  if (!blk.live) return;                           // padding of the grid (whole workgroup)
  const int seg = blk.seg, h = blk.h, b = blk.b;
  const int n_chunks = pr.T / C;
  const int c0 = seg * L, nc = min(L, n_chunks - c0);
  const long long sv_t = pr.sv[1];

  // Exclusive prefix (S_{<c}, Z_{<c}) of this segment: the scanned state at position seg, or
  // (sum_prefix) the states of segments 0 .. seg-1 added in that order; zero without states (one
  // segment per sequence).  Every wave keeps its own copy of Z (4 registers); lane holds
  // Z[4g + r][lane % 16].
  f32x4 S[LY::kSlots][4];
#pragma unroll
  for (int sl = 0; sl < LY::kSlots; ++sl)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) S[sl][nt] = zero4();
  f32x4 Z = zero4();
  static_assert(kPacked || !kCompact, "only packed states are stored compactly");
  {
    // the tile indices as scalars: the per-tile part of the places stays in scalar registers
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int n_stored = Stored<kPacked, GW>::floats(kCompact);
    const int z_stored = Stored<kPacked, GW>::zoff(kCompact);
    FragPlace<kPacked, GW, kCompact> fp[LY::kSlots];
#pragma unroll
    for (int sl = 0; sl < LY::kSlots; ++sl)
      if (LY::owns(wu, sl)) fp[sl].init(LY::tile(wu, sl), lane);
    auto add_state = [&](int j) {
      const float* pre = states + ((long long)(b * pr.H + h) * n_seg + j) * n_stored;
#pragma unroll
      for (int sl = 0; sl < LY::kSlots; ++sl) {
        if (!LY::owns(w, sl)) continue;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) fp[sl].add(pre, nt, S[sl][nt]);
      }
      Z += *reinterpret_cast<const f32x4*>(pre + z_stored + lane * 4);
    };
    const int j0 = sum_prefix ? 0 : seg, j1 = !states ? j0 : sum_prefix ? seg : seg + 1;
    int j = j0;
    if constexpr (kPacked)                         // two states' loads in flight
      for (; j + 1 < j1; j += 2) {
        add_state(j);
        add_state(j + 1);
      }
    for (; j < j1; ++j) add_state(j);
  }
  UpdateRows<kPacked, GW> ur;
  ur.init(w, lane);
  zero_pad_rows(tl, tid);

  // readout rows of this lane group: direct K step kk covers rows (2kk + r'/4, 4g + r'%4);
  // packed K step kk covers (a + r'/4, 4J + r'%4): (a, J) = ro_block(kk, g) at GW = 16, else the
  // double group 4kk + g of the grouped list
  constexpr bool kRo = kPacked && GW == P;
  int qa_off[LY::kSteps], qj_off[LY::kSteps];
#pragma unroll
  for (int kk = 0; kk < LY::kSteps; ++kk) {
    if (kRo) {
      qa_off[kk] = 2 * ro_block(kk, g).A;
      qj_off[kk] = 4 * ro_block(kk, g).J;
    } else if (kPacked) {
      int a, J;
      LY::dg(4 * kk + g, a, J);
      qa_off[kk] = a;
      qj_off[kk] = 4 * J;
    } else {
      qa_off[kk] = 2 * kk;
      qj_off[kk] = 4 * g;
    }
  }
  // where this lane's rows of each owned tile go in Sb: K step and lane (the tile's lane group
  // g holds the double group 4 (t >> 1) + g of the layout's list); half t & 1
  int pub_step[LY::kSlots], pub_lane[LY::kSlots];
#pragma unroll
  for (int sl = 0; sl < LY::kSlots; ++sl) {
    const int t = LY::owns(w, sl) ? LY::tile(w, sl) : 0;
    pub_step[sl] = t >> 1;
    pub_lane[sl] = lane;
    if (kRo) {
      int a, J;
      LY::dg(4 * (t >> 1) + g, a, J);
      const int pos = ro_slot(a >> 1, J);
      pub_step[sl] = pos >> 2;
      pub_lane[sl] = 16 * (pos & 3) + l16;
    }
  }

  // publish this wave's state tiles as bf16 MFMA operands: tile t fills slots 4 (t & 1) .. +3
  // of its rows' K step (slot r' <-> row 4g + r'%4 of tile 2(t>>1) + r'/4)
  auto publish = [&]() {
#pragma unroll
    for (int sl = 0; sl < LY::kSlots; ++sl) {
      if (!LY::owns(w, sl)) continue;
      const int t = LY::tile(w, sl);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (__bf16)S[sl][nt][r];
        reinterpret_cast<uint2*>(&sm.Sb[pub_step[sl]][nt][pub_lane[sl]])[t & 1] =
            __builtin_bit_cast(uint2, x);
      }
    }
  };

  // Each wave records whether the v rows it stages hold an infinity or a nan; the chunk's
  // masked P.V step then takes the slow exact path (nonfinite_fixup in mfma_util.h).
  auto flag_v = [&](const Stage& x) {
    const bool bad = (nonfinite_bf16x8(x.v0) | nonfinite_bf16x8(x.v1)) != 0u;
    const uint32_t any = __any(bad) ? 1u : 0u;
    if (lane == 0) sm.vbad[w] = any;
  };

  // Z as the bf16 hi + lo A operands of the q^T Z q products (KATA-Mg: only the
  // within-group blocks of Z enter q^T Z q)
  auto z_split = [&](const f32x4& Zr, s16x4& zhi, s16x4& zlo) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float zr = (GW == P || (4 * g + r) / GW == l16 / GW) ? Zr[r] : 0.f;
      const __bf16 hi = (__bf16)zr;
      zhi[r] = __builtin_bit_cast(short, hi);
      zlo[r] = __builtin_bit_cast(short, (__bf16)(zr - (float)hi));
    }
  };
  // packed layouts: wave 0 alone keeps Z and publishes its split once per chunk (wave 0 has the
  // least intra-chunk work)
  constexpr bool kFuse = kPacked;
  constexpr int kZWave = 0;
  auto publish_z = [&]() {
    if (!kFuse || w != kZWave) return;
    s16x4 zhi, zlo;
    z_split(Z, zhi, zlo);
    const uint2 a = __builtin_bit_cast(uint2, zhi), bb = __builtin_bit_cast(uint2, zlo);
    sm.Zb[lane] = uint4{a.x, a.y, bb.x, bb.y};
  };

  StagePtrs sp = stage_ptrs(pr, q, k, v, b, h, c0 * C, true, tid);
  Stage st;
  stage_load(st, sp, sv_t);
  stage_store(st, tl, true, tid);
  flag_v(st);
  publish();
  publish_z();
  __syncthreads();

  // output pointer of this lane's first store in the first chunk: token 16w + 8 (lane / 32),
  // column lane % 32
  Tout* orow = o + row_off(pr.so, b, c0 * C + 16 * w + 8 * (lane >> 5), h) + (lane & 31);
  const long long so_t = pr.so[1];

  for (int c = 0; c < nc; ++c) {
    const int tok0 = (c0 + c) * C;
    if (c + 1 < nc) {
      sp.next();
      stage_load(st, sp, sv_t);
    }
    const int t = 16 * w + l16;                  // this lane's token (fragment column / row)
    const uint4 vb4 = *reinterpret_cast<const uint4*>(sm.vbad);
    const bool vbad = __builtin_amdgcn_readfirstlane(vb4.x | vb4.y | vb4.z | vb4.w) != 0;

    // ---- intra-chunk tile of this wave's tokens, and (packed layouts) S += Phi(K)^T V with the
    // same value fragments: the readout reads the published S_{<c}, not these registers.  The
    // direct layout (4 tiles a wave) updates after the readout, for its register budget ----
    float lsum = 0.f;
    f32x4 O[4] = {zero4(), zero4(), zero4(), zero4()};
    const s16x4 qf = row4_frag(tl.Qs, 16 * w, lane);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (!kFuse && 2 * m > w) break;
      bf16x8 vb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) vb[nt] = v_frag(tl.V, m, nt, lane);
      if (kFuse) state_update_step<kPacked, GW>(tl, ur, S, vb, w, m, lane);
      if (2 * m > w) continue;                     // key tiles entirely in the future
      // the step holding the wave's diagonal tile (and any future keys) when a value of the
      // chunk is an infinity or a nan (rare, wave-uniform): exact path
      const bool fix = vbad && 2 * m + 1 >= w;
      uint32_t pw[2][2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ms = 2 * m + half;
        if (ms < w) {
          score_tile<GW, false>(row4_frag(tl.Ks, 16 * ms, lane), qf, lane, pw[half], lsum);
        } else if (ms == w) {
          score_tile<GW, true>(row4_frag(tl.Ks, 16 * ms, lane), qf, lane, pw[half], lsum);
        } else {
          pw[half][0] = pw[half][1] = 0u;
        }
      }
      const bf16x8 a = __builtin_bit_cast(bf16x8, uint4{pw[0][0], pw[0][1], pw[1][0], pw[1][1]});
      if (!fix) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) O[nt] = mfma32(a, vb[nt], O[nt]);
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) O[nt] = mfma32(a, finite_or_zero(vb[nt]), O[nt]);
        const int cols[4] = {l16, 16 + l16, 32 + l16, 48 + l16};
        nonfinite_fixup<4>(O, tl.V, a, 32 * m, 16 * w, cols, lane);
      }
    }

    // ---- inter-chunk denominator q^T Z_{<c} q ----
    // Y = Z q_t on MFMA with Z split into bf16 hi + lo (fp32-accurate; q is exact in bf16):
    // Z's accumulator layout (lane: column lane%16, rows 4g + r) is, Z being symmetric, the
    // A layout of a 16 x 16 x 16 product; q_t[4g..4g+3] is the same B operand as the scores.
    // Packed layouts: the split published by the wave that keeps Z (z_split, sm.Zb).
    float zq = 0.f;
    {
      s16x4 zhi, zlo;
      if constexpr (kFuse) {
        const uint4 zz = sm.Zb[lane];
        zhi = __builtin_bit_cast(s16x4, uint2{zz.x, zz.y});
        zlo = __builtin_bit_cast(s16x4, uint2{zz.z, zz.w});
      } else {
        z_split(Z, zhi, zlo);
      }
      f32x4 y = mfma16(zhi, qf, zero4());
      y = mfma16(zlo, qf, y);                   // y[r] = (Z q_t)[4g + r]
      const uint2 qq = __builtin_bit_cast(uint2, qf);
      zq = fmaf(bf_lo(qq.x), y[0], zq);
      zq = fmaf(bf_hi(qq.x), y[1], zq);
      zq = fmaf(bf_lo(qq.y), y[2], zq);
      zq = fmaf(bf_hi(qq.y), y[3], zq);
    }
    // the lane groups' shares of both sums at once; 1 / D_t from v_rcp_f32 (1 ulp)
    const float dsum = sum_xor32(sum_xor16(zq + lsum));
    if (g == 0) {
      const float D = pr.eps + dsum;
      sm.den[t] = D;
      sm.inv[t] = __builtin_amdgcn_rcpf(D);
    }

    // ---- readout phi(q_t)^T S_{<c} over all published state rows ----
    // (issue priority raised over the readout's MFMA stream: other waves' VALU work fills in)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < LY::kSteps; ++kk) {
      const uint32_t qa = *reinterpret_cast<const uint32_t*>(&tl.Qs[t][qa_off[kk]]);
      const uint2 qj = *reinterpret_cast<const uint2*>(&tl.Qs[t][qj_off[kk]]);
      const float i0 = bf_lo(qa), i1 = bf_hi(qa);
      const float jv[4] = {bf_lo(qj.x), bf_hi(qj.x), bf_lo(qj.y), bf_hi(qj.y)};
      bf16x8 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[r] = (__bf16)(i0 * jv[r]);
        a[4 + r] = (__bf16)(i1 * jv[r]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        O[nt] = mfma32(a, __builtin_bit_cast(bf16x8, sm.Sb[kk][nt][lane]), O[nt]);
    }

    __builtin_amdgcn_s_setprio(0);

    // ---- gate and store this wave's tokens: lane holds tokens 16w + 4g + r, column 16nt + l16.
    // Row-group swaps between column tiles 2j and 2j + 1 give each lane half a row of 32
    // consecutive columns, so every store writes two whole 128-byte rows (fp32) instead of
    // half rows of four tokens: the first register of a swap then holds tokens 16w + r (lanes
    // 0-31) and 16w + 8 + r (lanes 32-63), the second tokens 16w + 4 + r and 16w + 12 + r.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float inv = sm.inv[16 * w + 4 * g + r];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(O[2 * j][r] * inv),
                                                         __float_as_uint(O[2 * j + 1][r] * inv),
                                                         false, false);
        // streamed out: never re-read by this kernel
        __builtin_nontemporal_store(cvt_out<Tout>(__uint_as_float(sw[0])), orow + r * so_t + 32 * j);
        __builtin_nontemporal_store(cvt_out<Tout>(__uint_as_float(sw[1])),
                                    orow + (4 + r) * so_t + 32 * j);
      }
    }
    if (den_out && lane < 16)
      den_out[((long long)b * pr.T + tok0 + 16 * w + lane) * pr.H + h] = sm.den[16 * w + lane];
    orow += C * so_t;

    // ---- Z += K^T K (and S += Phi(K)^T V unless done with the intra-chunk tile) ----
    if (kFuse) {
      if (w == kZWave)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 kf = kcol_frag(tl, m, lane);
        Z = mfma32(kf, kf, Z);
      }
    } else {
      state_update<kPacked, GW>(tl, ur, S, Z, w, lane, true);
    }
    __syncthreads();                               // all reads of this chunk's tiles and Sb done
    if (c + 1 < nc) {
      stage_store(st, tl, true, tid);
      flag_v(st);
      publish();
      publish_z();
    }
    __syncthreads();
  }
}

}  // namespace

bool chunk_fast_available() { return true; }

namespace {
template <typename Tout, bool kPacked, int GW>
void walk_launch(const DevProblem& pr, const SegGrid& sg, int L, int n_seg, dim3 grid,
                 hipStream_t st, const __bf16* q, const __bf16* k, const __bf16* v, void* o,
                 float* den, const float* states, int sum_prefix) {
  if (kPacked && pr.stored_compact)
    launch_kernel(chunk_output_fast_kernel<Tout, kPacked, GW, kPacked>, grid, kThreads, 0, st,
        pr, sg, L, n_seg, q, k, v, (Tout*)o, den, states, sum_prefix);
  else
    launch_kernel(chunk_output_fast_kernel<Tout, kPacked, GW, false>, grid, kThreads, 0, st,
        pr, sg, L, n_seg, q, k, v, (Tout*)o, den, states, sum_prefix);
}

template <typename Tout>
void walk_dispatch(const DevProblem& pr, const SegGrid& sg, bool packed, int gw, int L, int n_seg,
                   dim3 grid, hipStream_t st, const __bf16* q, const __bf16* k, const __bf16* v,
                   void* o, float* den, const float* states, int sum_prefix) {
  if (gw == 8)
    walk_launch<Tout, true, 8>(pr, sg, L, n_seg, grid, st, q, k, v, o, den, states, sum_prefix);
  else if (gw == 4)
    walk_launch<Tout, true, 4>(pr, sg, L, n_seg, grid, st, q, k, v, o, den, states, sum_prefix);
  else if (packed)
    walk_launch<Tout, true, P>(pr, sg, L, n_seg, grid, st, q, k, v, o, den, states, sum_prefix);
  else
    walk_launch<Tout, false, P>(pr, sg, L, n_seg, grid, st, q, k, v, o, den, states, sum_prefix);
}
}  // namespace

// gw: group width (16, or 8 / 4 for KATA-Mg, which always use the packed layout)
hipError_t launch_chunk_state_fast(const DevProblem& pr, bool packed, int gw, int L, int n_seg,
                                   int n_used, const void* k, const void* v, float* states,
                                   hipStream_t st) {
  if (pr.p != P || pr.dv != DV || pr.C != C) return hipErrorInvalidValue;
  if (gw != P && gw != 8 && gw != 4) return hipErrorInvalidValue;
  const SegGrid sg = make_seg_grid(pr, n_seg);
  if (sg.blocks() > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)sg.blocks());
  const __bf16 *kk = (const __bf16*)k, *vv = (const __bf16*)v;
  if (gw == 8)
    launch_kernel(chunk_state_fast_kernel<true, 8>, grid, kThreads, 0, st, pr, sg, L, n_seg,
                  n_used, kk, vv, states);
  else if (gw == 4)
    launch_kernel(chunk_state_fast_kernel<true, 4>, grid, kThreads, 0, st, pr, sg, L, n_seg,
                  n_used, kk, vv, states);
  else if (packed)
    launch_kernel(chunk_state_hybrid_kernel, grid, kThreads, 0, st, pr, sg, L, n_seg, n_used,
                  kk, vv, states);
  else
    launch_kernel(chunk_state_dpp_kernel<false>, grid, kThreads, 0, st, pr, sg, L, n_seg,
                  n_used, kk, vv, states);
  return hipGetLastError();
}

hipError_t launch_chunk_output_fast(const DevProblem& pr, bool packed, int gw, bool out_bf16,
                                    int L, int n_seg, const void* q, const void* k,
                                    const void* v, void* o, float* den, const float* states,
                                    bool sum_prefix, hipStream_t st) {
  if (pr.p != P || pr.dv != DV || pr.C != C) return hipErrorInvalidValue;
  if (gw != P && gw != 8 && gw != 4) return hipErrorInvalidValue;
  const SegGrid sg = make_seg_grid(pr, n_seg);
  if (sg.blocks() > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)sg.blocks());
  const __bf16 *qq = (const __bf16*)q, *kk = (const __bf16*)k, *vv = (const __bf16*)v;
  if (out_bf16)
    walk_dispatch<__bf16>(pr, sg, packed, gw, L, n_seg, grid, st, qq, kk, vv, o, den, states,
                          sum_prefix);
  else
    walk_dispatch<float>(pr, sg, packed, gw, L, n_seg, grid, st, qq, kk, vv, o, den, states,
                         sum_prefix);
  return hipGetLastError();
}

}  // namespace kata

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
#include "device.h"
#include "kata.h"
#include "mfma_util.h"

namespace kata {
namespace {

constexpr int P = 16, DV = 64, C = 64, F = P * P;
constexpr int kThreads = 256;
constexpr int kStateFloats = F * (DV + 1);     // 16640: S (4 waves x 16 tiles x 256) + Z (256)
// LDS row strides, chosen so that every access pattern below is free of bank conflicts
// (32 banks of 4 bytes; 4-, 8- and 16-byte accesses served 32, 16 and 8 lanes at a time):
constexpr int QROW = 20;                       // bf16 per q / k row: 40 B, 8-byte aligned
constexpr int KTROW = 68;                      // fp32 per row of the K^T tile
constexpr int VROW = 80;                       // bf16 per v row: 160 B, 16-byte aligned

// ---- chunk tiles in LDS ------------------------------------------------------------------
// kPacked adds rows to the K^T tile: rows 16..31 hold 2 k (the weight of an off-diagonal
// packed state row) and row 32 zeros (the padding rows of the packed layout).
template <bool kPacked>
struct __align__(16) TilesT {
  __bf16 Qs[C][QROW];                 // q rows (bf16), row-major
  __bf16 Ks[C][QROW];                 // k rows (bf16), row-major
  float KT[kPacked ? 2 * P + 1 : P][KTROW];   // k transposed, fp32 (exact copies)
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
        tl.KT[P + 8 * half + 2 * e][row] = 2.f * lo;       // exact
        tl.KT[P + 8 * half + 2 * e + 1][row] = 2.f * hi;
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
// irow selects the K^T row for the i factor (i, 16 + i for the doubled copy, 32 for zeros).
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
// the A operand kf (k rows) and the B operand qf (q_t[4g .. 4g + 3]), masked and rounded to bf16
// P.  GW < 16 (KATA-Mg, groups of GW coordinates): one product per group, the query operand cut
// to the lane groups holding that group's coordinates, and the squared group dots summed.
template <int GW, bool kMask>
__device__ __forceinline__ void score_tile(const s16x4& kf, const s16x4& qf, int s0, int t,
                                           int lane, __bf16 out[4], float& lsum) {
  if constexpr (GW == P) {
    square_mask<kMask>(mfma16(kf, qf, zero4()), s0, t, lane, out, lsum);
  } else {
    const int grp = (4 * (lane >> 4)) / GW;
    f32x4 x2 = zero4();
#pragma unroll
    for (int j = 0; j < P / GW; ++j) {
      const s16x4 qj = grp == j ? qf : s16x4{0, 0, 0, 0};
      const f32x4 sc = mfma16(kf, qj, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) x2[r] = fmaf(sc[r], sc[r], x2[r]);
    }
    weight_mask<kMask>(x2, s0, t, lane, out, lsum);
  }
}

// ==========================================================================================
// Per-layout constants shared by the state and walk kernels.
//   direct: 16 state tiles (tile = i, rows j), wave w owns tiles 4w .. 4w+3, 8 readout K steps.
//   packed: the double groups of the unique pairs (see mfma_util.h), two per 16-row tile:
//           10 tiles at GW = 16, 5 readout K steps.  Wave w owns tiles w, w + 4, w + 8, so
//           waves 0-1 own 3 and waves 2-3 (more intra-chunk work) own 2.
//   KATA-Mg (packed, groups of GW = 8 or 4 consecutive coordinates): only the double groups
//           inside one group exist, 6 or 4 tiles.
// State layout in the workspace (floats): tile t, value tile nt, lane -> ((t*4 + nt)*64 +
// lane)*4 .. +3 (the accumulator registers as they are), then Z as one 16 x 16 tile.
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
        irow[sl] = i > j ? 2 * P : (i == j ? i : P + i);
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

template <bool kPacked>
__device__ __forceinline__ void zero_pad_rows(TilesT<kPacked>& tl, int tid) {
  if (kPacked && tid < KTROW) tl.KT[kPacked ? 2 * P : 0][tid] = 0.f;
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
  if (seg >= n_used) {
    // a state no prefix needs (the last segment's, in the forward): zeros for the scan, and
    // its k, v are not read
    float4* out = reinterpret_cast<float4*>(
        states + ((long long)(b * pr.H + h) * n_seg + seg) * LY::kStateFloats);
    for (int x = tid; x < LY::kStateFloats / 4; x += kThreads) out[x] = float4{0.f, 0.f, 0.f, 0.f};
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
  float* out = states + ((long long)(b * pr.H + h) * n_seg + seg) * LY::kStateFloats;
#pragma unroll
  for (int sl = 0; sl < LY::kSlots; ++sl) {
    if (!LY::owns(w, sl)) continue;
    const int t = LY::tile(w, sl);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      *reinterpret_cast<f32x4*>(out + ((t * 4 + nt) * 64 + lane) * 4) = S[sl][nt];
  }
  if (w == 0) *reinterpret_cast<f32x4*>(out + LY::kZOff + lane * 4) = Z;
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
template <bool kPacked, int GW>
struct __align__(16) WalkLds {
  TilesT<kPacked> tl;
  uint4 Sb[Layout<kPacked, GW>::kSteps][4][64];   // S_{<c} as MFMA operands: [K step][value tile][lane]
  float den[C];                               // D_t of the chunk's tokens
  float inv[C];                               // 1 / D_t
};

template <typename Tout, bool kPacked, int GW>
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
  {
    auto add_state = [&](int j) {
      const float* pre = states + ((long long)(b * pr.H + h) * n_seg + j) * LY::kStateFloats;
#pragma unroll
      for (int sl = 0; sl < LY::kSlots; ++sl) {
        if (!LY::owns(w, sl)) continue;
        const int t = LY::tile(w, sl);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          S[sl][nt] += *reinterpret_cast<const f32x4*>(pre + ((t * 4 + nt) * 64 + lane) * 4);
      }
      Z += *reinterpret_cast<const f32x4*>(pre + LY::kZOff + lane * 4);
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
  // packed K step m' covers (a + r'/4, 4J + r'%4) with (a, J) the double group 4m' + g
  int qa_off[LY::kSteps], qj_off[LY::kSteps];
#pragma unroll
  for (int kk = 0; kk < LY::kSteps; ++kk) {
    if (kPacked) {
      int a, J;
      LY::dg(4 * kk + g, a, J);
      qa_off[kk] = a;
      qj_off[kk] = 4 * J;
    } else {
      qa_off[kk] = 2 * kk;
      qj_off[kk] = 4 * g;
    }
  }

  // publish this wave's state tiles as bf16 MFMA operands: tile t fills slots 4 (t & 1) .. +3
  // of K step t >> 1 (slot r' of lane group g <-> row 4g + r'%4 of tile 2(t>>1) + r'/4)
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
        reinterpret_cast<uint2*>(&sm.Sb[t >> 1][nt][lane])[t & 1] = __builtin_bit_cast(uint2, x);
      }
    }
  };

  StagePtrs sp = stage_ptrs(pr, q, k, v, b, h, c0 * C, true, tid);
  Stage st;
  stage_load(st, sp, sv_t);
  stage_store(st, tl, true, tid);
  publish();
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
          score_tile<GW, false>(row4_frag(tl.Ks, 16 * ms, lane), qf, 16 * ms, t, lane,
                                &pa[4 * half], lsum);
        } else if (ms == w) {
          score_tile<GW, true>(row4_frag(tl.Ks, 16 * ms, lane), qf, 16 * ms, t, lane,
                               &pa[4 * half], lsum);
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
        // KATA-Mg: only the within-group blocks of Z enter q^T Z q
        const float zr = (GW == P || (4 * g + r) / GW == l16 / GW) ? Z[r] : 0.f;
        const __bf16 hi = (__bf16)zr;
        zhi[r] = __builtin_bit_cast(short, hi);
        zlo[r] = __builtin_bit_cast(short, (__bf16)(zr - (float)hi));
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

    // ---- readout phi(q_t)^T S_{<c} over all published state rows ----
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

    // ---- state update with this chunk: S += Phi(K)^T V, Z += K^T K ----
    state_update<kPacked, GW>(tl, ur, S, Z, w, lane, true);
    __syncthreads();                               // all reads of this chunk's tiles and Sb done
    if (c + 1 < nc) {
      stage_store(st, tl, true, tid);
      publish();
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
  launch_kernel(chunk_output_fast_kernel<Tout, kPacked, GW>, grid, kThreads, 0, st,
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
    launch_kernel(chunk_state_fast_kernel<true, P>, grid, kThreads, 0, st, pr, sg, L, n_seg,
                  n_used, kk, vv, states);
  else
    launch_kernel(chunk_state_fast_kernel<false, P>, grid, kThreads, 0, st, pr, sg, L, n_seg,
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

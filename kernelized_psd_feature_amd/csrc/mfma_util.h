// bf16 MFMA helpers shared by the gfx950 kernels of the chunked and quadratic forwards.
//
// MFMA fragment conventions (v_mfma_f32_16x16x32_bf16 / _16x16x16bf16_1k, wave64):
//   A (16 x K): lane l holds row l%16 and K-slots [KPL*(l/16), KPL*(l/16)+KPL)
//   B (K x 16): lane l holds column l%16 and the same K-slots
//   D (16 x 16 fp32): lane l holds column l%16, rows 4*(l/16) + r, r = 0..3
// A contraction only needs A and B to enumerate K in the same order, so the K order of every
// product over keys is chosen to match the D layout of the producing product ("slot kappa"):
// for a 32-wide K step m over keys, slot r' of lane group g is key 32m + 16*(r'/4) + 4g + r'%4.
// With that order the squared-score tile (computed transposed, keys as rows) is directly the A
// operand of P.V, and the fp32 state tiles are directly the B operand of the readout.
//
// Packed state rows ("double groups"): the unique feature pairs i <= j of a p-dimensional
// vec(u u^T) are listed in groups of 8 rows, double group (a, J) being the pairs
// (a + x, 4J + r) for x in {0, 1}, r in {0..3}, over J = 0 .. p/4 - 1 and even a <= 4J + 2.
// Every pair i <= j appears exactly once; the few pairs with i > j that the groups also list
// are zero rows.  Off the diagonal a row carries weight 2, since
// vec(q q^T) . vec(k k^T) = sum_i q_i^2 k_i^2 + 2 sum_{i<j} q_i q_j k_i k_j.  (The p = 32
// kernels order their rows differently, without most of the zero rows: fast32.hip.)
#pragma once

#include "device.h"

namespace kata {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint4 ld16(const __bf16* p) { return *reinterpret_cast<const uint4*>(p); }

// B operand of a 32-key step m for value columns [16 nt, 16 nt + 16), slot order kappa, read
// from a row-major V tile with two LDS transpose loads.  Within a 16-lane block, lane i's
// slot r of ds_read_b64_tr_b16 is element (i % 4) of the 8 bytes addressed by block lane
// 4r + i/4; block lane j therefore points at V[key(g, j/4)][16 nt + 4 (j % 4)], which hands
// lane i the value V[key(g, r)][16 nt + i].
template <int ROW>
__device__ __forceinline__ bf16x8 v_frag(const __bf16 (*V)[ROW], int m, int nt, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int row = 32 * m + 4 * g + (j >> 2), col = 16 * nt + 4 * (j & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&V[row][col]));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&V[row + 16][col]));
  const uint2 ul = __builtin_bit_cast(uint2, lo), uh = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, uint4{ul.x, ul.y, uh.x, uh.y});
}

// Double group idx -> (a, J): the groups of column block J are indices J (J + 1) ..
// J (J + 1) + 2J + 1, one for each even a = 0, 2, .., 4J + 2.  p = 16 has 20 groups.
__device__ __forceinline__ void double_group(int idx, int& a, int& J) {
  J = 0;
  while ((J + 1) * (J + 2) <= idx) ++J;
  a = 2 * (idx - J * (J + 1));
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

// As square_mask for a tile of weights that are already sums of squares (KATA-Mg).
template <bool kMask>
__device__ __forceinline__ void weight_mask(const f32x4& x2, int s0, int t, int lane,
                                            __bf16 out[4], float& lsum) {
  const int g = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    __bf16 pb = (__bf16)x2[r];
    if (kMask) pb = (s0 + 4 * g + r <= t) ? pb : (__bf16)0.f;
    out[r] = pb;
    lsum += (float)pb;
  }
}

template <typename Tout>
__device__ __forceinline__ Tout cvt_out(float x) { return from_f32<Tout>(x); }

// Two floats rounded to bf16 (round to nearest even) and packed, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f2;
  typedef __attribute__((ext_vector_type(2))) __bf16 b2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
}
// acc + lo(w) + hi(w) for a packed bf16 pair w (v_dot2 with ones, fp32 accumulation).
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 b2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w),
                                         __builtin_bit_cast(b2, 0x3f803f80u), acc, false);
}

// x + x(lane ^ 16) and x + x(lane ^ 32) in every lane, from the row-swap permutes (no LDS
// round trip).  Swapping a register with a copy of itself leaves the two 16-lane rows of each
// pair in the two results, so their sum is the pair sum in both rows (the same value the two
// orders of an IEEE add give).
__device__ __forceinline__ float sum_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// ---- non-finite values and masked P.V products ------------------------------------------
// Inside an MFMA P.V product a masked weight P_ts = 0 still meets the value v_s of every key of
// the K step, and 0 * inf or 0 * nan is nan: a non-finite value of a later token would reach
// earlier outputs of the same tile.  The kernels therefore check the values of a tile; when one
// is non-finite, the tile's masked steps take the value operand with those entries replaced by
// zero (so masked pairs add exact zeros, as they do for finite values) and add the exact
// contributions of the non-finite entries of unmasked pairs afterwards, pair by pair.

// Bit 15 (bit 31) of the result is set when the low (high) bf16 of w is an infinity or a nan:
// the magnitude |h| = h & 0x7fff is >= 0x7f80 exactly then, so |h| + 0x80 reaches 0x8000, and
// the low half (at most 0x807f) never carries into the high half.
__device__ __forceinline__ uint32_t nonfinite_bf16x2(uint32_t w) {
  return ((w & 0x7fff7fffu) + 0x00800080u) & 0x80008000u;
}
__device__ __forceinline__ uint32_t nonfinite_bf16x8(const uint4& u) {
  return nonfinite_bf16x2(u.x) | nonfinite_bf16x2(u.y) | nonfinite_bf16x2(u.z) |
         nonfinite_bf16x2(u.w);
}
__device__ __forceinline__ bool nonfinite_bf16(__bf16 x) {
  return nonfinite_bf16x2(__builtin_bit_cast(unsigned short, x)) != 0u;
}
// w with every non-finite bf16 replaced by +0
__device__ __forceinline__ uint32_t finite_or_zero_bf16x2(uint32_t w) {
  return w & ~((nonfinite_bf16x2(w) >> 15) * 0xffffu);
}
__device__ __forceinline__ bf16x8 finite_or_zero(const bf16x8& x) {
  const uint4 u = __builtin_bit_cast(uint4, x);
  return __builtin_bit_cast(bf16x8, uint4{finite_or_zero_bf16x2(u.x), finite_or_zero_bf16x2(u.y),
                                          finite_or_zero_bf16x2(u.z), finite_or_zero_bf16x2(u.w)});
}

// After a walk step's P.V product over keys [s0, s0 + 32) was taken with finite_or_zero value
// operands: O[n][r] (query row 4 (lane / 16) + r of the wave's 16 tokens, whose chunk-local token
// is t0 + 4 (lane / 16) + r, value column cols[n]) += P[row][s] * V[s][cols[n]] for every key
// s <= that token whose value is non-finite.  pa: the step's bf16 weights as the P.V A operand
// (lane holds query row lane % 16, keys s0 + 16 (i / 4) + 4 (lane / 16) + i % 4 in slot i); the
// weight of another row is fetched from the lane that holds it.  V: the row-major value tile of
// the chunk.  Called by all lanes of the wave (the shuffles need them).
template <int NT, int ROW>
__device__ __forceinline__ void nonfinite_fixup(f32x4 (&O)[NT], const __bf16 (*V)[ROW],
                                                const bf16x8& pa, int s0, int t0,
                                                const int (&cols)[NT], int lane) {
  const int g = lane >> 4;
  const uint4 pd = __builtin_bit_cast(uint4, pa);
  for (int j = 0; j < 32; ++j) {
    const int s = s0 + j;
    if (s > t0 + 15) break;                        // past the wave's last token (uniform)
    const int slot = 4 * (j >> 4) + (j & 3);       // wave-uniform
    const uint32_t d = slot < 2 ? pd.x : slot < 4 ? pd.y : slot < 6 ? pd.z : pd.w;
    const int src = 16 * ((j & 15) >> 2) + 4 * g;  // + r: the lane holding row 4 g + r
    float w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t x = (uint32_t)__shfl((int)d, src + r);
      w[r] = (slot & 1) ? bf_hi(x) : bf_lo(x);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const __bf16 x = V[s][cols[n]];
      if (!nonfinite_bf16(x)) continue;
      const float xf = (float)x;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (s <= t0 + 4 * g + r) O[n][r] += w[r] * xf;
    }
  }
}

}  // namespace kata

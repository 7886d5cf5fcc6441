// Associative prefix scan over chunk states for gfx950.
//
// The states of one sequence form an [n][elems] fp32 array; the scan runs independently for
// every element.  Because the state update is additive and commutative (ai.info Main
// Findings, readout-gate bullet), the associative operator is addition, and the scan is a
// tree of depth ceil(log2 n) (gist.science section 2.3: inter-chunk depth O(N_C) ->
// O(log N_C)).  Two forms:
//
// scan_short_kernel (n <= 64): one lane per row, the tree across the lanes of a wave by DPP
// moves (see below).
//
// scan_tile_kernel (tiles of up to 256 rows, Kogge-Stone): one workgroup takes one sequence,
// one tile of rows and a strip of `strip` coordinates (a multiple of 4, so every access is a
// float4; for strip = 64 a wave reads four whole 256-byte rows per instruction).  The tile is
// held in two LDS buffers: each tree level writes the thread's float4 slots to one buffer,
// synchronizes, and adds the slot 2^l rows up; alternating buffers needs a single barrier per
// level.
#include "device.h"

namespace kata {
namespace {

constexpr int kScanThreads = 256;
constexpr int kMaxSlots = 16;   // float4 slots per thread: 256 threads * 16 * 4 = 16384 floats

// kSlots: float4 slots per thread, a power of two >= ceil(tile_rows * strip / 4 / 256), so the
// per-thread loops run no more iterations than the tile needs.
template <int kSlots>
__global__ __launch_bounds__(kScanThreads) void scan_tile_kernel(
    float* __restrict__ x, long long n, long long elems, int strip, int tile_rows,
    int n_tiles, int exclusive, float* __restrict__ totals,
    const float* __restrict__ tile_offsets) {
  extern __shared__ float4 lds[];
  const int sv = strip / 4;                       // float4 slots per row
  const long long seq = blockIdx.z;
  const int tile = blockIdx.y;
  // Consecutive workgroups go to consecutive XCDs (8), each with its own L2.  When a strip's
  // row piece is narrower than a 128-byte line, the strips sharing a line get ids congruent
  // mod 8, so one XCD fetches each line once (a bijection of [0, gridDim.x)).
  long long sx = blockIdx.x;
  const int per_line = 32 / strip;                // strips per 128-byte line of one row
  if (per_line > 1 && gridDim.x % (8 * per_line) == 0) {
    const long long id = blockIdx.x, blk = id / (8 * per_line);
    sx = (blk * 8 + id % 8) * per_line + (id / 8) % per_line;
  }
  const long long col0 = sx * strip;
  const long long r0 = (long long)tile * tile_rows;
  const int nr = (int)min((long long)tile_rows, n - r0);
  const int nslots = nr * sv;
  float4* buf0 = lds;
  float4* buf1 = lds + (long long)tile_rows * sv;
  float* base = x + (seq * n + r0) * elems + col0;

  float4 val[kSlots];
  int rowv[kSlots];
#pragma unroll
  for (int m = 0; m < kSlots; ++m) {
    const int slot = threadIdx.x + m * kScanThreads;
    const int r = slot / sv, cv = slot % sv;
    rowv[m] = r;
    const bool ok = slot < nslots && col0 + cv * 4 < elems;
    val[m] = ok ? *reinterpret_cast<const float4*>(base + (long long)r * elems + cv * 4)
                : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // Kogge-Stone levels: x[r] += x[r - 2^l]
  int lvl = 0;
  for (int off = 1; off < nr; off <<= 1, ++lvl) {
    float4* buf = (lvl & 1) ? buf1 : buf0;
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
      const int slot = threadIdx.x + m * kScanThreads;
      if (slot < nslots) buf[slot] = val[m];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
      const int slot = threadIdx.x + m * kScanThreads;
      if (slot < nslots && rowv[m] >= off) {
        const float4 y = buf[slot - off * sv];
        val[m].x += y.x; val[m].y += y.y; val[m].z += y.z; val[m].w += y.w;
      }
    }
  }
  // val = inclusive prefix within the tile; add the tile's exclusive offset
  if (tile_offsets) {
    const float* ob = tile_offsets + (seq * n_tiles + tile) * elems + col0;
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
      const int slot = threadIdx.x + m * kScanThreads;
      const int cv = slot % sv;
      if (slot < nslots && col0 + cv * 4 < elems) {
        const float4 y = *reinterpret_cast<const float4*>(ob + cv * 4);
        val[m].x += y.x; val[m].y += y.y; val[m].z += y.z; val[m].w += y.w;
      }
    }
  }
  const bool last_tile = (tile == n_tiles - 1);
  if (totals && last_tile) {
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
      const int slot = threadIdx.x + m * kScanThreads;
      const int cv = slot % sv;
      if (slot < nslots && rowv[m] == nr - 1 && col0 + cv * 4 < elems)
        *reinterpret_cast<float4*>(totals + seq * elems + col0 + cv * 4) = val[m];
    }
  }
  if (exclusive) {
    // exclusive[r] = inclusive[r - 1]; row 0 takes the tile offset (or zero)
    float4* buf = (lvl & 1) ? buf1 : buf0;
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
      const int slot = threadIdx.x + m * kScanThreads;
      if (slot < nslots) buf[slot] = val[m];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
      const int slot = threadIdx.x + m * kScanThreads;
      const int cv = slot % sv;
      if (slot < nslots && col0 + cv * 4 < elems) {
        float4 y;
        if (rowv[m] > 0) {
          y = buf[slot - sv];
        } else if (tile_offsets) {
          y = *reinterpret_cast<const float4*>(
              tile_offsets + (seq * n_tiles + tile) * elems + col0 + cv * 4);
        } else {
          y = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        val[m] = y;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < kSlots; ++m) {
    const int slot = threadIdx.x + m * kScanThreads;
    const int cv = slot % sv;
    if (slot < nslots && col0 + cv * 4 < elems)
      *reinterpret_cast<float4*>(base + (long long)rowv[m] * elems + cv * 4) = val[m];
  }
}

// Sum of the rows of each tile: sums[seq][tile][e].  Grid (ceil(elems/256/4), n_tiles, n_seq).
__global__ __launch_bounds__(kScanThreads) void tile_sums_kernel(
    const float* __restrict__ x, long long n, long long elems, int tile_rows, int n_tiles,
    float* __restrict__ sums) {
  const long long seq = blockIdx.z;
  const int tile = blockIdx.y;
  const long long e = ((long long)blockIdx.x * kScanThreads + threadIdx.x) * 4;
  if (e >= elems) return;
  const long long r0 = (long long)tile * tile_rows;
  const int nr = (int)min((long long)tile_rows, n - r0);
  const float* p = x + (seq * n + r0) * elems + e;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int r = 0; r < nr; ++r) {
    const float4 y = *reinterpret_cast<const float4*>(p + (long long)r * elems);
    acc.x += y.x; acc.y += y.y; acc.z += y.z; acc.w += y.w;
  }
  *reinterpret_cast<float4*>(sums + (seq * n_tiles + tile) * elems + e) = acc;
}

// ---- scans of at most 64 rows --------------------------------------------------------------
// A workgroup takes a strip of 64 coordinates of one sequence: the rows are read coalesced
// (a wave covers four whole 256-byte row pieces per instruction) into an LDS tile, then each
// wave takes 16 of the coordinates with one lane per row and builds the tree across its lanes
// with DPP moves: row_shr 1, 2, 4 and 8 inside each 16-lane row, then row_bcast:15 joins rows
// 0-1 and 2-3 and row_bcast:31 joins the halves.  Level l adds the partial sum 2^l lanes back
// (inside a row) or the last partial of the row block before, so after ceil(log2 n) levels (the
// ones a shorter scan needs) every lane holds its inclusive prefix; the exclusive one is a wave
// shift by one lane.  The results go back through the tile and out coalesced: two barriers
// instead of one per level.
constexpr int kShortRows = 64;
constexpr int kShortStrip = 64;                    // coordinates per workgroup
constexpr int kShortRow = kShortStrip + 4;         // LDS row stride (floats): conflict-free
constexpr int kShortThreads = 256;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float x) {
  // lanes whose source lies outside the pattern (bound_ctrl) or whose row is masked off get 0
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, true));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_level(float4 (&v)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j].x += dpp_or_zero<CTRL, ROW_MASK>(v[j].x);
    v[j].y += dpp_or_zero<CTRL, ROW_MASK>(v[j].y);
    v[j].z += dpp_or_zero<CTRL, ROW_MASK>(v[j].z);
    v[j].w += dpp_or_zero<CTRL, ROW_MASK>(v[j].w);
  }
}

__global__ __launch_bounds__(kShortThreads) void scan_short_kernel(
    float* __restrict__ x, long long n, long long elems, int exclusive, float* __restrict__ totals) {
  __shared__ float4 tile[kShortRows * kShortRow / 4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const long long seq = blockIdx.y;
  const long long col0 = (long long)blockIdx.x * kShortStrip;
  float* base = x + seq * n * elems + col0;
  constexpr int kVec = kShortStrip / 4;            // float4 per row piece
  const int nv = (int)n * kVec;
  // rows in: thread s takes row s / 16, float4 s % 16
  for (int s = tid; s < nv; s += kShortThreads) {
    const int r = s / kVec, c = s % kVec;
    if (col0 + 4 * c < elems)
      tile[r * (kShortRow / 4) + c] = *reinterpret_cast<const float4*>(base + r * elems + 4 * c);
  }
  __syncthreads();
  // wave w: coordinates 16 w .. 16 w + 15 of the strip, lane = row
  const bool row_ok = lane < n;
  float4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    v[j] = row_ok ? tile[lane * (kShortRow / 4) + 4 * w + j] : make_float4(0.f, 0.f, 0.f, 0.f);
  // DPP controls: row_shr:k = 0x110 + k, row_bcast:15 = 0x142, row_bcast:31 = 0x143
  if (n > 1) scan_level<0x111, 0xF>(v);
  if (n > 2) scan_level<0x112, 0xF>(v);
  if (n > 4) scan_level<0x114, 0xF>(v);
  if (n > 8) scan_level<0x118, 0xF>(v);
  if (n > 16) scan_level<0x142, 0xA>(v);           // rows 1 and 3 take lane 15 of the row before
  if (n > 32) scan_level<0x143, 0xC>(v);           // rows 2 and 3 take lane 31
  if (totals && lane == n - 1) {
    float* tp = totals + seq * elems + col0 + 16 * w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (col0 + 16 * w + 4 * j < elems) *reinterpret_cast<float4*>(tp + 4 * j) = v[j];
  }
  if (exclusive) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {                  // wave_shr:1 = 0x138; lane 0 gets 0
      v[j].x = dpp_or_zero<0x138, 0xF>(v[j].x);
      v[j].y = dpp_or_zero<0x138, 0xF>(v[j].y);
      v[j].z = dpp_or_zero<0x138, 0xF>(v[j].z);
      v[j].w = dpp_or_zero<0x138, 0xF>(v[j].w);
    }
  }
  __syncthreads();                                 // every row read before any is overwritten
  if (row_ok) {
#pragma unroll
    for (int j = 0; j < 4; ++j) tile[lane * (kShortRow / 4) + 4 * w + j] = v[j];
  }
  __syncthreads();
  for (int s = tid; s < nv; s += kShortThreads) {
    const int r = s / kVec, c = s % kVec;
    if (col0 + 4 * c < elems)
      *reinterpret_cast<float4*>(base + r * elems + 4 * c) = tile[r * (kShortRow / 4) + c];
  }
}

}  // namespace

hipError_t launch_scan_short(float* x, long long n_seq, long long n, long long elems,
                             int exclusive, float* totals, hipStream_t st) {
  if (n < 1 || n > kShortRows || n_seq < 1 || n_seq > 65535) return hipErrorInvalidValue;
  const long long blocks = (elems + kShortStrip - 1) / kShortStrip;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks, (unsigned)n_seq);
  launch_kernel(scan_short_kernel, grid, kShortThreads, 0, st, x, n, elems, exclusive, totals);
  return hipGetLastError();
}

hipError_t launch_scan_tiles(float* x, long long n_seq, long long n, long long elems,
                             int strip, int tile_rows, int n_tiles, int exclusive,
                             float* totals, const float* tile_offsets, hipStream_t st) {
  // every slot of the tile must fit the per-thread register array
  if ((long long)tile_rows * (strip / 4) > (long long)kScanThreads * kMaxSlots)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)((elems + strip - 1) / strip), n_tiles, (unsigned)n_seq);
  size_t lds = 2 * (size_t)tile_rows * (strip / 4) * sizeof(float4);
  const long long slots = ((long long)tile_rows * (strip / 4) + kScanThreads - 1) / kScanThreads;
  int ks = 1;
  while (ks < slots) ks <<= 1;
  auto go = [&](auto kern) -> hipError_t {
    // up to 128 KiB of the 160 KiB LDS of a gfx950 CU
    hipError_t e = ensure_dynamic_lds((const void*)kern, 131072);
    if (e != hipSuccess) return e;
    launch_kernel(kern, grid, kScanThreads, lds, st, x, n, elems, strip, tile_rows, n_tiles,
                  exclusive, totals, tile_offsets);
    return hipSuccess;
  };
  hipError_t e;
  switch (ks) {
    case 1: e = go(scan_tile_kernel<1>); break;
    case 2: e = go(scan_tile_kernel<2>); break;
    case 4: e = go(scan_tile_kernel<4>); break;
    case 8: e = go(scan_tile_kernel<8>); break;
    default: e = go(scan_tile_kernel<16>); break;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_tile_sums(const float* x, long long n_seq, long long n, long long elems,
                            int tile_rows, int n_tiles, float* sums, hipStream_t st) {
  dim3 grid((unsigned)((elems / 4 + kScanThreads - 1) / kScanThreads), n_tiles,
            (unsigned)n_seq);
  launch_kernel(tile_sums_kernel, grid, kScanThreads, 0, st, x, n, elems, tile_rows, n_tiles, sums);
  return hipGetLastError();
}

}  // namespace kata

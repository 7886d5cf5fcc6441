// Associative prefix scan over chunk states for gfx950.
//
// The states of one sequence form an [n][elems] fp32 array; the scan runs independently for
// every element.  Because the state update is additive and commutative (ai.info Main
// Findings, readout-gate bullet), the associative operator is addition, and the scan is a
// Kogge-Stone tree of depth ceil(log2 n) (gist.science section 2.3: inter-chunk depth
// O(N_C) -> O(log N_C)).
//
// One workgroup takes one sequence, one tile of rows and a strip of `strip` coordinates
// (a multiple of 4, so every access is a float4; for strip = 64 a wave reads four whole
// 256-byte rows per instruction).  The tile is held in two LDS buffers: each tree level
// writes the thread's float4 slots to one buffer, synchronizes, and adds the slot 2^l rows
// up; alternating buffers needs a single barrier per level.
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

}  // namespace

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

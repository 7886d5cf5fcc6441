// Device-side helpers shared by the gfx950 kernels, and the launcher declarations the host
// API calls.  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace kata {

// ---- kernel launch -------------------------------------------------------------------
// The open per-kernel timing scope of this host thread (null when timing is off): a pair of
// events that the scope's first launch stamps with its start and every launch with its end.
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
LaunchTiming* launch_timing();

// Every kernel of the library is launched here.  With timing on, the launch goes through
// hipExtLaunchKernelGGL so the events take the timestamps of the kernel's own dispatch: no
// marker packets are enqueued between kernels, and the recorded time is the kernels' alone.
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t st,
                          Args... args) {
  LaunchTiming* t = launch_timing();
  if (t) {
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)shmem, st,
                          t->used ? nullptr : t->start, t->stop, 0u, args...);
    t->used = true;
  } else {
    kernel<<<grid, block, shmem, st>>>(args...);
  }
}

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once per (kernel,
// device) in the process -- the attribute stays set -- so that launches after the first pay a
// table lookup, not a runtime call.  Returns the runtime's error if setting it fails.
hipError_t ensure_dynamic_lds(const void* kernel, int bytes);

// Problem description passed to kernels by value.
struct DevProblem {
  int B, H, T, p, dv, C;
  int gs;                                          // KATA-Mg group width (p: one group)
  int stored_compact;                              // packed p = 16 segment states stored
                                                   // without their zero rows (scan plans)
  float eps;
  long long sq[3], sk[3], sv[3], so[3], sdo[3];   // element strides of (b, t, h)
};

// ---- segment grids: one workgroup per (segment, head, batch) -------------------------
// Consecutive workgroup ids are dispatched to consecutive XCDs, each with its own L2.  In
// (B, T, H, D) storage the q and k rows of `hg` neighbouring heads share 128-byte lines, so
// the workgroups of such a line group (same batch and segment) get ids congruent mod 8: one
// XCD then fetches each line once.  Line groups are enumerated (batch, segment) first, so
// when B * n_seg is a multiple of 8 every line group of one (batch, segment) lands on the same
// XCD too (whole token rows per XCD), and the XCDs get equal shares.  The grid is
// one-dimensional, padded to a multiple of 8 line groups; padding workgroups exit at once.
struct SegGrid {
  int n_seg, hg, n_hgrp;      // segments, heads per line group, line groups per (b, segment)
  long long bs;               // B * n_seg
  long long groups;           // bs * n_hgrp
  long long blocks() const { return ((groups + 7) / 8) * 8 * hg; }
};

inline SegGrid make_seg_grid(const DevProblem& pr, int n_seg) {
  SegGrid g;
  g.n_seg = n_seg;
  const bool heads_adjacent = pr.sq[2] == pr.p && pr.sk[2] == pr.p;
  g.hg = heads_adjacent ? (64 / pr.p > 1 ? 64 / pr.p : 1) : 1;   // 2p bytes per bf16 row
  g.n_hgrp = (pr.H + g.hg - 1) / g.hg;
  g.bs = (long long)pr.B * n_seg;
  g.groups = g.bs * g.n_hgrp;
  return g;
}

struct SegBlock {
  int seg, h, b;
  bool live;
};

__device__ __forceinline__ SegBlock seg_block(const SegGrid& g, int H) {
  const long long x = blockIdx.x, xcd = x % 8, r = x / 8;
  const long long gi = (r / g.hg) * 8 + xcd;       // line group
  const long long bs = gi % g.bs;
  SegBlock s;
  s.h = int((gi / g.bs) * g.hg + r % g.hg);
  s.seg = int(bs % g.n_seg);
  s.b = int(bs / g.n_seg);
  s.live = gi < g.groups && s.h < H;
  return s;
}

// ---- KATA-Mg scores ------------------------------------------------------------------
// The p coordinates form groups of gs consecutive entries; the score of a (query, key) pair
// is the sum over groups of the squared group dot product (a single group: (q . k)^2), and
// the feature pair (i, j) exists only within a group.  Bit i of `start` / `last` marks the
// first / last coordinate of a group, so the loops below stay fully unrolled.
struct Groups {
  unsigned start, last;
};

__device__ __forceinline__ Groups make_groups(int p, int gs) {
  Groups g{0u, 0u};
  for (int i = 0; i < p; ++i) {
    if (i % gs == 0) g.start |= 1u << i;
    if (i % gs == gs - 1) g.last |= 1u << i;
  }
  return g;
}

__device__ __forceinline__ bool same_group(int i, int j, int gs) { return i / gs == j / gs; }

// sum over groups of (x . y restricted to the group)^2
template <int P, typename Y>
__device__ __forceinline__ float grouped_square(const float (&x)[P], const Y& y, Groups g) {
  float a = 0.f, run = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    run = fmaf(x[i], y[i], ((g.start >> i) & 1u) ? 0.f : run);
    if ((g.last >> i) & 1u) a = fmaf(run, run, a);
  }
  return a;
}

// As grouped_square, and sc[i] = the dot product of coordinate i's group.
template <int P, typename Y>
__device__ __forceinline__ float grouped_dots(const float (&x)[P], const Y& y, Groups g,
                                              float (&sc)[P]) {
  float cum[P];
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    run = fmaf(x[i], y[i], ((g.start >> i) & 1u) ? 0.f : run);
    cum[i] = run;
  }
  float a = 0.f, cur = 0.f;
#pragma unroll
  for (int i = P - 1; i >= 0; --i) {
    if ((g.last >> i) & 1u) {
      cur = cum[i];
      a = fmaf(cur, cur, a);
    }
    sc[i] = cur;
  }
  return a;
}

__device__ __forceinline__ long long row_off(const long long* s, int b, int t, int h) {
  return (long long)b * s[0] + (long long)t * s[1] + (long long)h * s[2];
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }   // RNE

// ---- launchers (defined in the .hip files) --------------------------------------------
// in_bf16 / out_bf16 select the element types; every launcher returns hipGetLastError().

hipError_t launch_quadratic_generic(const DevProblem& pr, bool in_bf16, bool out_bf16,
                                    const void* q, const void* k, const void* v, void* o,
                                    float* den, hipStream_t st);

hipError_t launch_chunk_state_generic(const DevProblem& pr, bool in_bf16, const void* k,
                                      const void* v, float* states, int n_chunks,
                                      hipStream_t st);

hipError_t launch_chunk_output_generic(const DevProblem& pr, bool in_bf16, bool out_bf16,
                                       const void* q, const void* k, const void* v, void* o,
                                       float* den, const float* states, int n_chunks,
                                       hipStream_t st);

// Prefix scan of n <= 64 rows per sequence (one lane per row, the tree across a wave).
hipError_t launch_scan_short(float* x, long long n_seq, long long n, long long elems,
                             int exclusive, float* totals, hipStream_t st);

// Prefix scan of one tile-level: rows [tile*tile_rows, ...) of every sequence, `strip`
// coordinates per workgroup.  tile_offsets (nullable) holds the exclusive offset of each
// tile, [n_seq][n_tiles][elems].
hipError_t launch_scan_tiles(float* x, long long n_seq, long long n, long long elems,
                             int strip, int tile_rows, int n_tiles, int exclusive,
                             float* totals, const float* tile_offsets, hipStream_t st);

hipError_t launch_tile_sums(const float* x, long long n_seq, long long n, long long elems,
                            int tile_rows, int n_tiles, float* sums, hipStream_t st);

hipError_t launch_decode(const DevProblem& pr, bool in_bf16, bool out_bf16, const void* q,
                         const void* k, const void* v, void* o, float* den, float* state,
                         hipStream_t st);
hipError_t launch_state_sum(const float* src, long long n_seq, long long n, long long elems,
                            bool tiles, float* dst, hipStream_t st);
hipError_t launch_bwd_chunk_prep(const DevProblem& pr, bool in_bf16, const void* dO, float* g,
                                 float* e, hipStream_t st);
hipError_t launch_bwd_chunk_dq(const DevProblem& pr, bool in_bf16, const void* q, const void* k,
                               const void* v, const float* g, const float* e,
                               const float* states, int n_chunks, float* dq, hipStream_t st);
hipError_t launch_bwd_rev_state(const DevProblem& pr, bool in_bf16, const void* q,
                                const float* g, const float* e, float* states, int n_chunks,
                                hipStream_t st);
hipError_t launch_bwd_chunk_dkdv(const DevProblem& pr, bool in_bf16, const void* q,
                                 const void* k, const void* v, const float* g, const float* e,
                                 const float* states, int n_chunks, float* dk, float* dv,
                                 hipStream_t st);
hipError_t launch_bwd_prep(const DevProblem& pr, bool in_bf16, const void* q, const void* k,
                           const void* v, const void* dO, float* D, float* delta,
                           hipStream_t st);
hipError_t launch_bwd_dq(const DevProblem& pr, bool in_bf16, const void* q, const void* k,
                         const void* v, const void* dO, const float* D, const float* delta,
                         float* dq, hipStream_t st);
hipError_t launch_bwd_dkdv(const DevProblem& pr, bool in_bf16, const void* q, const void* k,
                           const void* v, const void* dO, const float* D, const float* delta,
                           float* dk, float* dv, hipStream_t st);

}  // namespace kata

// Host-side argument validation and launch planning.  Pure C++ (no HIP): it is compiled into
// libkata.so and, on its own with tests/plan_fuzz.cpp, into a CPU fuzz driver built with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_plan_sanitizers.py).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "kata.h"

namespace kata {

enum class Form { Quadratic, Chunked, Backward };

// Most segments per sequence for which the p = 32 state pass is spread (ChunkPlan::sp).
constexpr int kSpreadMaxSegments = 4;

// Most segments per sequence for which the walks form their prefixes without a scan.
constexpr int kWalkPrefixMaxSegments = 8;

// Which kernels run a chunked forward, and the workspace they need.
struct ChunkPlan {
  int fast = 0;               // 1: bf16 MFMA kernels; 0: fp32-arithmetic VALU kernels
  int fast32 = 0;             // 1: the MFMA kernels are the p = 32 ones (always packed)
  int packed = 0;             // 1: the MFMA kernels keep the unique (i <= j) state rows
  int gw = 16;                // p = 16 MFMA kernels: KATA-Mg group width (16 = one group)
  int L = 1;                  // chunks per segment
  int n_chunks = 0;           // N_c = T / C per (b, h)
  int n_seg = 0;              // ceil(N_c / L)
  int walk_sums_prefix = 0;   // 1: each walk adds the earlier segments' states itself, no scan
  int compact = 0;            // 1: packed p = 16 states stored without their zero rows (scan)
  // p = 32, walks adding the prefixes themselves, at most 4 segments: the state pass spreads
  // the (n_seg - 1) L chunks that enter a prefix evenly over n_seg workgroups per sequence, sp
  // chunks each, and every workgroup leaves up to two states (the sum of its range, and of the
  // part before the segment boundary it crosses).  0: one workgroup and one state per segment.
  int sp = 0;
  // 1: p = 32 KATA-Mg (g >= 2) as two p = 16 passes over the coordinate halves (every other
  // field then describes one pass); the workspace adds the passes' fp32 outputs and D_t
  int halves = 0;
  size_t half_out_bytes = 0;  // one pass's fp32 output [B][T][H][dv], rounded up to 256
  size_t half_den_bytes = 0;  // one pass's D_t [B][T][H], rounded up to 256
  int dv_split = 1;           // workgroups sharing one segment, each owning dv / dv_split columns
  int64_t n_seq = 0;          // B * H
  int64_t state_elems = 0;    // floats in one segment state: p^2 (dv + 1)
  size_t states_bytes = 0;    // n_seq * n_seg * (sp ? 2 : 1) * state_elems * 4, rounded to 256
  size_t scan_ws_bytes = 0;   // extra workspace of the prefix scan over n_seg segments
  size_t ws_bytes = 0;        // total
};

// Prefix-scan tiling: a single Kogge-Stone tree when the chunk count fits one LDS tile, else
// tiles of `tile_rows` rows whose totals are scanned recursively.
struct ScanPlan {
  int64_t n_seq = 0, n = 0, elems = 0;
  int64_t tile_rows = 0;      // rows one workgroup scans in LDS
  int64_t strip = 0;          // coordinates per workgroup
  int64_t n_tiles = 0;        // ceil(n / tile_rows)
  size_t ws_bytes = 0;        // tile totals (recursive), 0 for a single tile
  int levels = 0;             // depth of the combining tree
  bool wave = false;          // n <= kScanWaveRows: one lane per row, the tree across a wave
};

constexpr int64_t kScanWaveRows = 64;   // rows of the wave form (one per lane)

constexpr int64_t kMaxT = int64_t(1) << 26;
constexpr int64_t kScanLdsFloats = 16384;   // per buffer; two buffers = 128 KiB of LDS

size_t elem_size(int32_t dtype);
bool dtype_pair_ok(int32_t in, int32_t out, Form f);

// Checks sizes, dtypes, eps and strides.  Returns KATA_OK or an error with `why` filled in.
kata_status validate_problem(const kata_problem* pr, Form f, std::string* why);

// Checks that a tensor's base pointer and strides keep every row 16-byte aligned.
kata_status validate_tensor(const void* ptr, const int64_t st[3], size_t esize,
                            const char* name, std::string* why);

// Checks the sizes of a stand-alone prefix scan (kata_chunk_state_scan): n_seq in
// [1, 65535], n in [1, 2^26], elems a positive multiple of 4 up to 2^30, and the states array,
// n_seq * n * elems fp32 values, below 2^62 bytes (so every size and offset derived from it
// fits 64 bits).  Returns KATA_OK or INVALID_ARGUMENT with `why` filled in.
kata_status validate_scan(int64_t n_seq, int64_t n, int64_t elems, std::string* why);

// Plan of the prefix scan; the sizes must have passed validate_scan (or come from a valid
// problem's plan).
ScanPlan plan_scan(int64_t n_seq, int64_t n, int64_t elems);
// pr must have passed validate_problem; fast_available: the MFMA chunked kernels are built.
ChunkPlan plan_chunked(const kata_problem* pr, bool fast_available);
// The same plan with one state per segment in the p = 32 state pass (sp = 0: half the states'
// workspace), for callers bound to a fixed scratch size.
ChunkPlan plan_unspread(ChunkPlan cp);

// Floats in one packed p = 32 segment state (34 tiles of 16 x 64 plus Z as four 16 x 16 tiles).
constexpr int64_t kState32Floats = 34 * 16 * 64 + 4 * 256;
size_t bwd_workspace_bytes(const kata_problem* pr);

}  // namespace kata

// Host-side argument validation and launch planning (pure C++, no HIP).
#include "plan.h"

#include <algorithm>
#include <cmath>

namespace kata {

namespace {

kata_status fail(std::string* why, kata_status s, const std::string& msg) {
  if (why) *why = msg;
  return s;
}

bool in_set(int32_t x, std::initializer_list<int32_t> s) {
  for (int32_t y : s)
    if (x == y) return true;
  return false;
}

int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

int ceil_log2(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace

size_t elem_size(int32_t dtype) {
  return dtype == KATA_F32 ? 4 : dtype == KATA_BF16 ? 2 : 0;
}

bool dtype_pair_ok(int32_t in, int32_t out, Form f) {
  if (in != KATA_F32 && in != KATA_BF16) return false;
  if (f == Form::Backward) return true;                 // gradients are always fp32
  if (in == KATA_F32) return out == KATA_F32;
  return out == KATA_F32 || out == KATA_BF16;
}

kata_status validate_problem(const kata_problem* pr, Form f, std::string* why) {
  if (!pr) return fail(why, KATA_ERR_INVALID_ARGUMENT, "problem pointer is null");
  if (pr->B < 1 || pr->H < 1 || pr->T < 1)
    return fail(why, KATA_ERR_INVALID_ARGUMENT, "B, H and T must be >= 1");
  if (pr->T > kMaxT) return fail(why, KATA_ERR_UNSUPPORTED, "T exceeds 2^26");
  if (int64_t(pr->B) * pr->H > 65535)
    return fail(why, KATA_ERR_UNSUPPORTED, "B*H exceeds 65535");
  if (pr->p < 1 || pr->dv < 1)
    return fail(why, KATA_ERR_INVALID_ARGUMENT, "p and dv must be >= 1");
  if (!in_set(pr->p, {8, 16, 32}))
    return fail(why, KATA_ERR_UNSUPPORTED, "p must be 8, 16 or 32");
  if (!in_set(pr->dv, {16, 64}))
    return fail(why, KATA_ERR_UNSUPPORTED, "dv must be 16 or 64");
  if (pr->groups < 0 || pr->groups > pr->p || (pr->groups > 1 && pr->p % pr->groups))
    return fail(why, KATA_ERR_INVALID_ARGUMENT, "groups must be 0, 1 or a divisor of p");
  if (!std::isfinite(pr->eps) || pr->eps < 0.0f)
    return fail(why, KATA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (!dtype_pair_ok(pr->in_dtype, pr->out_dtype, f))
    return fail(why, KATA_ERR_INVALID_ARGUMENT,
                "dtype pair must be bf16->fp32, bf16->bf16 or fp32->fp32");
  if (f == Form::Chunked) {
    if (pr->chunk < 1) return fail(why, KATA_ERR_INVALID_ARGUMENT, "chunk must be >= 1");
    if (!in_set(pr->chunk, {16, 32, 64}))
      return fail(why, KATA_ERR_UNSUPPORTED, "chunk must be 16, 32 or 64");
    if (pr->T % pr->chunk)
      return fail(why, KATA_ERR_UNSUPPORTED, "T must be a multiple of chunk");
    if (pr->seg_chunks < 0)
      return fail(why, KATA_ERR_INVALID_ARGUMENT, "seg_chunks must be >= 0");
    if (pr->state_layout != KATA_STATE_DIRECT && pr->state_layout != KATA_STATE_PACKED)
      return fail(why, KATA_ERR_INVALID_ARGUMENT, "state_layout must be DIRECT or PACKED");
  }
  const int64_t* strides[5] = {pr->sq, pr->sk, pr->sv, pr->so, pr->sdo};
  const char* names[5] = {"q", "k", "v", "o", "dO"};
  const int64_t last[5] = {pr->p, pr->p, pr->dv, pr->dv, pr->dv};
  const int64_t sizes[3] = {pr->B, pr->T, pr->H};
  for (int i = 0; i < 5; ++i) {
    if (i == 4 && f != Form::Backward) continue;
    // every (b, t, h) row must start past the previous row's last element along some order;
    // the minimal check that catches swapped or zero strides: each stride of an axis with
    // more than one entry is >= the row length.
    // the largest element offset, sum_a (size_a - 1) stride_a + row length, in bytes must stay
    // below 2^62 so that every offset the kernels form in 64-bit arithmetic is exact
    const int64_t kMaxExtent = int64_t(1) << 62;
    int64_t extent = last[i];
    for (int a = 0; a < 3; ++a) {
      int64_t s = strides[i][a];
      if (s < 0) return fail(why, KATA_ERR_INVALID_ARGUMENT, std::string(names[i]) + ": negative stride");
      if (sizes[a] > 1 && s < last[i])
        return fail(why, KATA_ERR_INVALID_ARGUMENT,
                    std::string(names[i]) + ": stride smaller than the row length");
      if (sizes[a] > 1 && s > (kMaxExtent - extent) / (sizes[a] - 1))
        return fail(why, KATA_ERR_INVALID_ARGUMENT,
                    std::string(names[i]) + ": strides address more than 2^62 elements");
      extent += (sizes[a] - 1) * s;
    }
    if (extent > kMaxExtent / 4)
      return fail(why, KATA_ERR_INVALID_ARGUMENT,
                  std::string(names[i]) + ": strides address more than 2^62 bytes");
  }
  return KATA_OK;
}

kata_status validate_tensor(const void* ptr, const int64_t st[3], size_t esize,
                            const char* name, std::string* why) {
  if (!ptr) return fail(why, KATA_ERR_INVALID_ARGUMENT, std::string(name) + " is null");
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    return fail(why, KATA_ERR_INVALID_ARGUMENT, std::string(name) + " is not 16-byte aligned");
  for (int a = 0; a < 3; ++a)
    if ((uint64_t(st[a]) * esize) % 16)
      return fail(why, KATA_ERR_INVALID_ARGUMENT,
                  std::string(name) + ": stride is not a multiple of 16 bytes");
  return KATA_OK;
}

kata_status validate_scan(int64_t n_seq, int64_t n, int64_t elems, std::string* why) {
  if (n_seq < 1 || n < 1 || elems < 4 || elems % 4)
    return fail(why, KATA_ERR_INVALID_ARGUMENT,
                "need n_seq >= 1, n_chunks >= 1, state_elems >= 4 and a multiple of 4");
  if (n_seq > 65535 || n > kMaxT || elems > (int64_t(1) << 30))
    return fail(why, KATA_ERR_INVALID_ARGUMENT, "scan sizes out of range");
  // n_seq * n < 2^42 here; the array's bytes must stay below 2^62
  if (n_seq * n > ((int64_t(1) << 60) - 1) / elems)
    return fail(why, KATA_ERR_INVALID_ARGUMENT, "states array exceeds 2^62 bytes");
  return KATA_OK;
}

ScanPlan plan_scan(int64_t n_seq, int64_t n, int64_t elems) {
  ScanPlan sp;
  sp.n_seq = n_seq;
  sp.n = n;
  sp.elems = elems;
  if (n <= 0 || n_seq <= 0 || elems <= 0) return sp;
  if (n <= kScanWaveRows) {
    // strips of 64 coordinates, one lane per row, ceil(log2 n) DPP levels
    sp.wave = true;
    sp.tile_rows = n;
    sp.strip = 64;
    sp.n_tiles = 1;
    sp.ws_bytes = 0;
    sp.levels = ceil_log2(n);
    return sp;
  }
  int64_t np2 = next_pow2(n);
  if (np2 * 4 <= kScanLdsFloats) {
    // one tree over all n rows; a strip of at least 64 coordinates, widened for short scans
    // so that a workgroup moves about 2048 floats (few rows would otherwise leave most of
    // its threads idle; wider strips cost parallelism), and at most what the LDS tile holds.
    // From 2048 rows on, half the LDS (4 coordinates at 2048 rows), so that two workgroups
    // share a CU and one loads or stores while the other runs its tree: the 2048-state scan
    // at 131k tokens (16 sequences) 1.85 -> 1.30 ms, bitwise the same.
    const int64_t cap = np2 >= 2048 ? std::max<int64_t>(4, kScanLdsFloats / 2 / np2)
                                    : kScanLdsFloats / np2;
    int64_t strip = ((2048 / n + 63) / 64) * 64;
    if (strip < 64) strip = 64;
    if (strip > cap) strip = cap;
    sp.strip = strip;
    sp.tile_rows = n;
    sp.n_tiles = 1;
    sp.ws_bytes = 0;
    sp.levels = ceil_log2(n);
    return sp;
  }
  // tiles of 256 rows; their totals are scanned by a recursive plan
  sp.tile_rows = 256;
  sp.strip = 64;
  sp.n_tiles = (n + sp.tile_rows - 1) / sp.tile_rows;
  ScanPlan sub = plan_scan(n_seq, sp.n_tiles, elems);
  sp.ws_bytes = round256(size_t(n_seq) * size_t(sp.n_tiles) * size_t(elems) * 4) + sub.ws_bytes;
  // tile sums (tree, log2 tile) -> scan of the totals -> tile tree + offset add
  sp.levels = 2 * ceil_log2(sp.tile_rows) + sub.levels + 1;
  return sp;
}

// Segment length when the walks add their earlier segments' states themselves (2 ..
// kWalkPrefixMaxSegments segments per sequence, one round of walks).  The last segment's walk
// is the longest: L chunks of token data plus n - 1 states.  Among the segment counts that
// still fill two thirds of the slots, take the one whose last walk moves the fewest bytes
// (ties: the most segments).  At 8 x 16 heads x 2048 tokens (32 chunks): 4 segments of 8
// chunks, 0.051 ms per step against 0.0525 ms for 6 of 6; at 8 x 16 x 4096 it keeps 6.  Not
// for the p = 32 kernels: their walk is bound by its MFMAs, one workgroup per CU, and fewer
// segments leave CUs idle (4 x 16 x 1024: 3 segments 0.058 ms, 4 segments 0.054 ms).
static int walk_sum_segment_length(const kata_problem* pr, const ChunkPlan& cp, int64_t slots,
                                   int L) {
  const int64_t n0 = (cp.n_chunks + L - 1) / L;
  if (cp.fast32 || n0 < 2 || n0 > kWalkPrefixMaxSegments || cp.n_seq * n0 > slots) return L;
  const int64_t out_bytes = pr->out_dtype == KATA_BF16 ? 2 : 4;
  const int64_t chunk_bytes =
      int64_t(pr->chunk) * (2 * (2 * int64_t(pr->p) + pr->dv) + out_bytes * pr->dv);
  const int64_t state_bytes = cp.state_elems * 4;
  int best_L = L;
  int64_t best = int64_t(L) * chunk_bytes + (n0 - 1) * state_bytes;
  for (int64_t s = n0 - 1; s >= 2; --s) {
    const int Ls = int((cp.n_chunks + s - 1) / s);
    const int64_t n = (cp.n_chunks + Ls - 1) / Ls;
    if (3 * cp.n_seq * n < 2 * slots) break;
    const int64_t cost = int64_t(Ls) * chunk_bytes + (n - 1) * state_bytes;
    if (cost < best) {
      best = cost;
      best_L = Ls;
    }
  }
  return best_L;
}

// States, scan workspace and total of a plan whose kernels are chosen (not the KATA-Mg halves).
static void set_workspace(ChunkPlan& cp) {
  const size_t per_seg = cp.sp ? 2 : 1;
  cp.states_bytes =
      round256(size_t(cp.n_seq) * size_t(cp.n_seg) * per_seg * size_t(cp.state_elems) * 4);
  cp.scan_ws_bytes =
      cp.walk_sums_prefix ? 0 : plan_scan(cp.n_seq, cp.n_seg, cp.state_elems).ws_bytes;
  cp.ws_bytes = cp.states_bytes + cp.scan_ws_bytes;
}

ChunkPlan plan_chunked(const kata_problem* pr, bool fast_available) {
  // p = 32 KATA-Mg on the MFMA kernels: the groups (16, 8 or 4 coordinates) lie inside the two
  // 16-coordinate halves, so a_ts is the sum of the halves' grouped scores; each half is a
  // p = 16 problem with g / 2 groups, run by the p = 16 kernels, and the two passes' numerators
  // and denominators are added.
  const int g32 = pr->groups <= 1 ? 1 : pr->groups;
  if (fast_available && pr->p == 32 && (g32 == 2 || g32 == 4 || g32 == 8) &&
      pr->in_dtype == KATA_BF16 && pr->dv == 64 && pr->chunk == 64) {
    kata_problem half = *pr;
    half.p = 16;
    half.groups = g32 / 2;
    half.out_dtype = KATA_F32;
    ChunkPlan cp = plan_chunked(&half, fast_available);
    const size_t n_tok = size_t(pr->B) * size_t(pr->T) * size_t(pr->H);
    cp.halves = 1;
    cp.half_out_bytes = round256(n_tok * size_t(pr->dv) * 4);
    cp.half_den_bytes = round256(n_tok * 4);
    cp.ws_bytes = round256(cp.ws_bytes) + 2 * (cp.half_out_bytes + cp.half_den_bytes);
    return cp;
  }
  ChunkPlan cp;
  cp.n_chunks = pr->T / pr->chunk;
  cp.n_seq = int64_t(pr->B) * pr->H;
  cp.state_elems = int64_t(pr->p) * pr->p * (pr->dv + 1);
  // MFMA kernels: bf16, d_v = 64, C = 64; p = 16 with g in {1, 2, 4} (group widths 16, 8,
  // 4), or p = 32 with g = 1
  const bool mfma_shape = fast_available && pr->in_dtype == KATA_BF16 && pr->dv == 64 &&
                          pr->chunk == 64;
  const int g = pr->groups <= 1 ? 1 : pr->groups;
  cp.fast = (mfma_shape && ((pr->p == 16 && (g == 1 || g == 2 || g == 4)) ||
                            (pr->p == 32 && g == 1))) ? 1 : 0;
  cp.fast32 = (cp.fast && pr->p == 32) ? 1 : 0;
  cp.gw = pr->p / g;
  if (cp.fast) {
    cp.packed = (pr->state_layout == KATA_STATE_PACKED || cp.fast32 || g > 1) ? 1 : 0;
    // packed: 10 tiles of 16 rows (the 136 unique (i, j) rows and 24 zero rows) x 64 columns,
    // plus the full 16 x 16 Z; KATA-Mg at p = 16: 6 tiles (g = 2) or 4 (g = 4), the
    // within-group pairs only; p = 32: 34 tiles (528 unique rows and 16 zero rows) and Z.
    // Through the scan the p = 16 states are stored without their zero rows (below).
    if (cp.packed) {
      const int tiles16 = g == 1 ? 10 : g == 2 ? 6 : 4;
      cp.state_elems = cp.fast32 ? kState32Floats : int64_t(tiles16) * 16 * 64 + 256;
    }
    int L = pr->seg_chunks;
    if (L == 0) {
      // With one walk per sequence filling at least two thirds of the workgroup slots of the
      // GPU (256 CUs x 3 resident workgroups; the p = 32 walk is one eight-wave workgroup per
      // CU: 256 slots), one segment per sequence: no segment states (which cost a second read
      // of k and v) and no scan.  Otherwise fill the slots in as few whole rounds as possible,
      // with segments of at most 64 chunks: fewer, longer segments mean less prefix-scan
      // traffic, whole rounds avoid an idle tail.  (Measured at 131072 tokens: 256 sequences
      // of 8192 run faster as 3 segments each, 512 of 4096 as one.)
      const int64_t slots = cp.fast32 ? 256 : 768;
      L = 1;
      if (3 * cp.n_seq >= 2 * slots) {
        L = cp.n_chunks;
      } else if (cp.n_seq * cp.n_chunks > slots) {
        for (int64_t rounds = 1;; ++rounds) {
          const int64_t seg_target = (rounds * slots) / cp.n_seq;
          if (seg_target < 1) continue;
          L = int((cp.n_chunks + seg_target - 1) / seg_target);
          if (L <= 64) break;
        }
        L = walk_sum_segment_length(pr, cp, slots, L);
      }
    }
    if (L > cp.n_chunks) L = cp.n_chunks;
    cp.L = L;
  } else {
    cp.L = 1;   // the VALU path scans every chunk state
  }
  cp.n_seg = (cp.n_chunks + cp.L - 1) / cp.L;
  // Few segments per sequence (MFMA kernels): the walk of segment s adds the states of
  // segments 0 .. s-1 itself.  That reads n(n-1)/2 states per sequence; the scan reads and
  // writes all n and the walks read n prefixes again, 3n, and costs a launch of its own.
  cp.walk_sums_prefix =
      (cp.fast && cp.n_seg >= 2 && cp.n_seg <= kWalkPrefixMaxSegments) ? 1 : 0;
  // Packed p = 16 states that go through the scan are stored without the tiles' zero rows:
  // the unique (i, j) rows of each group of gw coordinates, 16 (gw + 1) / 2 of them (136 at
  // g = 1, 72 at g = 2, 40 at g = 4) x 64 columns, plus Z, 15 % fewer bytes written, scanned
  // and read.  Walks that add the states themselves keep whole fragments (16-byte loads).
  cp.compact =
      (cp.fast && cp.packed && !cp.fast32 && cp.n_seg >= 2 && !cp.walk_sums_prefix) ? 1 : 0;
  if (cp.compact) cp.state_elems = int64_t(16) * (cp.gw + 1) / 2 * 64 + 256;
  // The p = 32 state pass otherwise runs n_seg - 1 of its n_seg workgroups per sequence (one
  // workgroup per CU): with 4 segments a quarter of the GPU idles.  Spread, every workgroup
  // takes sp = ceil((n_seg - 1) L / n_seg) chunks, and the walk of segment s adds up to s + 1
  // range sums (the last one cut at its start) instead of s states.  Beyond 4 segments the
  // idle share is small and the walks' extra state reads outweigh it.
  if (cp.fast32 && cp.walk_sums_prefix && cp.n_seg <= kSpreadMaxSegments)
    cp.sp = int((int64_t(cp.n_seg - 1) * cp.L + cp.n_seg - 1) / cp.n_seg);
  set_workspace(cp);
  return cp;
}

ChunkPlan plan_unspread(ChunkPlan cp) {
  if (cp.sp == 0) return cp;
  cp.sp = 0;
  set_workspace(cp);
  return cp;
}

size_t bwd_workspace_bytes(const kata_problem* pr) {
  // D_t and delta_t, fp32 [B][H][T] each
  return 2 * round256(size_t(pr->B) * pr->H * pr->T * 4);
}

}  // namespace kata

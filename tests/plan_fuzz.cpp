// Host fuzz driver for the library's pure-C++ argument validation and launch planning
// (kernelized_psd_feature_amd/csrc/plan.cpp), built by tests/test_plan_sanitizers.py with g++
// and AddressSanitizer + UndefinedBehaviorSanitizer (no HIP, no GPU).
//
//   plan_fuzz <seed> <iterations>
//
// Each iteration draws a kata_problem from a seeded generator -- sizes, dtypes, layouts,
// group counts, eps and strides over their valid ranges, their edges and far beyond them
// (negative, zero, 2^26 + 64, B * H = 65536, INT32/INT64 extremes, NaN/Inf eps, odd and huge
// strides) -- and runs validate_problem for every form, validate_tensor, plan_chunked (with
// and without the MFMA kernels), plan_scan and bwd_workspace_bytes.  Besides the sanitizers'
// own checks (out-of-bounds access, signed overflow, invalid shifts or conversions), it
// asserts the documented contracts: the status is one of the five codes, with a message on
// error; a valid problem respects every cap; an accepted tensor's largest byte offset stays
// below 2^62; and every plan of a valid problem is consistent, its byte counts equal to the
// exact products (computed in 128-bit arithmetic, so a wrapped size_t is caught).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include <limits>
#include <string>

#include "kata.h"
#include "plan.h"

namespace {

using u128 = unsigned __int128;
using i128 = __int128;

uint64_t g_state;
uint64_t next_u64() {   // splitmix64
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
template <typename T>
T pick(std::initializer_list<T> xs) {
  return *(xs.begin() + next_u64() % xs.size());
}
int64_t uniform(int64_t lo, int64_t hi) {   // inclusive
  return lo + int64_t(next_u64() % uint64_t(hi - lo + 1));
}
int32_t clamp32(int64_t x) {
  if (x > std::numeric_limits<int32_t>::max()) return std::numeric_limits<int32_t>::max();
  if (x < std::numeric_limits<int32_t>::min()) return std::numeric_limits<int32_t>::min();
  return int32_t(x);
}
int64_t sat64(i128 x) {
  const i128 m = std::numeric_limits<int64_t>::max();
  return int64_t(x > m ? m : x < -m ? -m : x);
}

const kata_problem* g_pr = nullptr;
[[noreturn]] void fail(const char* what) {
  const kata_problem& pr = *g_pr;
  std::fprintf(stderr,
               "FAIL %s: B=%d H=%d T=%d p=%d dv=%d chunk=%d seg=%d layout=%d groups=%d eps=%g "
               "in=%d out=%d sq=(%lld,%lld,%lld)\n",
               what, pr.B, pr.H, pr.T, pr.p, pr.dv, pr.chunk, pr.seg_chunks, pr.state_layout,
               pr.groups, double(pr.eps), pr.in_dtype, pr.out_dtype, (long long)pr.sq[0],
               (long long)pr.sq[1], (long long)pr.sq[2]);
  std::exit(1);
}
#define CHECK(cond, what) \
  do {                    \
    if (!(cond)) fail(what); \
  } while (0)

int64_t size_value() {
  switch (next_u64() % 4) {
    case 0: return uniform(1, 8);
    case 1: return uniform(1, 4096);
    case 2:
      return pick<int64_t>({0, 1, -1, 65535, 65536, 1 << 20, (1 << 26) - 64, 1 << 26,
                            (1 << 26) + 64, std::numeric_limits<int32_t>::max(),
                            std::numeric_limits<int32_t>::min()});
    default: return int64_t(next_u64());
  }
}

void draw_strides(const kata_problem& pr, int64_t last, int64_t out[3]) {
  // contiguous (B, T, H, D), head-major (B, H, T, D) storage, or arbitrary values
  const i128 T = pr.T, H = pr.H;
  switch (next_u64() % 4) {
    case 0: out[0] = sat64(T * H * last); out[1] = sat64(H * last); out[2] = last; break;
    case 1: out[0] = sat64(H * T * last); out[1] = last; out[2] = sat64(T * last); break;
    case 2:
      for (int a = 0; a < 3; ++a)
        out[a] = pick<int64_t>({0, -8, last, last + 8, 8 * last, int64_t(1) << 40,
                                int64_t(1) << 61, std::numeric_limits<int64_t>::max(),
                                std::numeric_limits<int64_t>::min(), 7});
      break;
    default:
      for (int a = 0; a < 3; ++a) out[a] = int64_t(next_u64() >> uniform(0, 63));
  }
}

kata_problem draw() {
  kata_problem pr{};
  const bool sane = next_u64() % 3 != 0;    // two thirds: mostly valid problems
  pr.B = clamp32(sane ? pick<int64_t>({1, 2, 4, 8, 64, 256}) : size_value());
  pr.H = clamp32(sane ? pick<int64_t>({1, 3, 16, 64, 255}) : size_value());
  pr.T = clamp32(sane ? pick<int64_t>({1, 64, 256, 1000, 2048, 131072, 1 << 26}) : size_value());
  pr.p = clamp32(sane ? pick<int64_t>({8, 16, 32}) : pick<int64_t>({0, -1, 4, 8, 16, 24, 32, 64, 1 << 30}));
  pr.dv = clamp32(sane ? pick<int64_t>({16, 64}) : pick<int64_t>({0, -1, 16, 32, 64, 128}));
  pr.chunk = clamp32(sane ? pick<int64_t>({16, 32, 64}) : pick<int64_t>({0, -1, 1, 16, 48, 64, 128}));
  pr.seg_chunks = clamp32(pick<int64_t>({0, 0, 1, 3, 43, 64, 4096, -1,
                                         std::numeric_limits<int32_t>::max()}));
  pr.state_layout = clamp32(pick<int64_t>({0, 1, 1, -1, 2}));
  pr.groups = clamp32(sane ? pick<int64_t>({0, 1, 2, 4, 8}) : pick<int64_t>({-1, 0, 3, 5, 16, 32, 33}));
  pr.eps = sane ? 1e-6f
                : pick<float>({0.f, 1e-6f, -1e-6f, 1e30f, std::numeric_limits<float>::infinity(),
                               std::numeric_limits<float>::quiet_NaN(),
                               std::numeric_limits<float>::denorm_min()});
  pr.in_dtype = clamp32(sane ? pick<int64_t>({0, 1, 1}) : pick<int64_t>({-1, 0, 1, 2}));
  pr.out_dtype = clamp32(sane ? pick<int64_t>({0, 0, 1}) : pick<int64_t>({-1, 0, 1, 2}));
  draw_strides(pr, pr.p, pr.sq);
  draw_strides(pr, pr.p, pr.sk);
  draw_strides(pr, pr.dv, pr.sv);
  draw_strides(pr, pr.dv, pr.so);
  draw_strides(pr, pr.dv, pr.sdo);
  return pr;
}

u128 round256(u128 b) { return (b + 255) / 256 * 256; }

int ceil_log2(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

// the largest byte offset a (b, t, h) row of `last` elements reaches with these strides
i128 extent_bytes(const kata_problem& pr, const int64_t st[3], int64_t last, int64_t esize) {
  const int64_t sizes[3] = {pr.B, pr.T, pr.H};
  i128 e = last;
  for (int a = 0; a < 3; ++a) e += i128(sizes[a] - 1) * st[a];
  return e * esize;
}

void check_scan(int64_t n_seq, int64_t n, int64_t elems) {
  const kata::ScanPlan sp = kata::plan_scan(n_seq, n, elems);
  if (n <= 0 || n_seq <= 0 || elems <= 0) return;
  CHECK(sp.n_tiles >= 1 && sp.tile_rows >= 1, "scan tiles");
  CHECK(i128(sp.n_tiles) * sp.tile_rows >= n, "scan tiles cover the rows");
  CHECK(sp.levels >= ceil_log2(n) && sp.levels <= 256, "scan depth");
  CHECK(sp.strip >= 1, "scan strip");
  CHECK(sp.wave == (n <= kata::kScanWaveRows), "wave form exactly for n <= 64 rows");
  if (sp.n_tiles == 1) {
    CHECK(sp.ws_bytes == 0 && sp.tile_rows == n, "single-tile scan");
    CHECK(sp.levels == ceil_log2(n), "single-tile scan depth");
    int64_t np2 = 1;
    while (np2 < n) np2 <<= 1;
    CHECK(sp.strip * np2 <= kata::kScanLdsFloats, "scan tile fits its LDS buffer");
  } else {
    CHECK(u128(sp.ws_bytes) >= round256(u128(n_seq) * u128(sp.n_tiles) * u128(elems) * 4),
          "scan workspace holds the tile totals");
  }
}

void check_chunked(const kata_problem& pr, bool fast) {
  const kata::ChunkPlan cp = kata::plan_chunked(&pr, fast);
  if (cp.halves) {    // p = 32 KATA-Mg: every other field describes one p = 16 pass
    CHECK(fast && pr.p == 32, "two-pass plan only for p = 32 on the MFMA kernels");
    const u128 tok = u128(pr.B) * u128(pr.T) * u128(pr.H);
    CHECK(u128(cp.half_out_bytes) == round256(tok * u128(pr.dv) * 4), "two-pass output bytes");
    CHECK(u128(cp.half_den_bytes) == round256(tok * 4), "two-pass den bytes");
    CHECK(cp.ws_bytes >= 2 * (cp.half_out_bytes + cp.half_den_bytes), "two-pass workspace");
    return;
  }
  CHECK(cp.n_chunks == pr.T / pr.chunk, "n_chunks");
  CHECK(cp.n_seq == int64_t(pr.B) * pr.H, "n_seq");
  CHECK(cp.L >= 1 && cp.L <= cp.n_chunks, "segment length");
  CHECK(cp.n_seg == (cp.n_chunks + cp.L - 1) / cp.L, "segment count");
  CHECK(cp.state_elems >= 4 && cp.state_elems % 4 == 0 &&
            cp.state_elems <= int64_t(pr.p) * pr.p * (pr.dv + 1),
        "state size");
  if (!cp.fast) {
    CHECK(cp.L == 1 && cp.state_elems == int64_t(pr.p) * pr.p * (pr.dv + 1), "fp32 plan");
    CHECK(!cp.walk_sums_prefix, "fp32 plan scans");
  }
  if (cp.fast) CHECK(pr.in_dtype == KATA_BF16 && pr.dv == 64 && pr.chunk == 64, "MFMA shape");
  if (cp.walk_sums_prefix)
    CHECK(cp.n_seg >= 2 && cp.n_seg <= kata::kWalkPrefixMaxSegments, "walk-summed prefix");
  if (cp.sp) {
    // spread p = 32 state pass: n_seg ranges of sp chunks cover the (n_seg - 1) L chunks before
    // the last segment, each range crosses at most one segment boundary
    CHECK(cp.fast32 && cp.walk_sums_prefix && cp.n_seg <= kata::kSpreadMaxSegments, "spread plan");
    CHECK(cp.sp >= 1 && cp.sp <= cp.L, "spread range length");
    CHECK(int64_t(cp.sp) * cp.n_seg >= int64_t(cp.n_seg - 1) * cp.L &&
              int64_t(cp.sp - 1) * cp.n_seg < int64_t(cp.n_seg - 1) * cp.L,
          "spread ranges cover the prefix chunks, the shortest such length");
    const kata::ChunkPlan un = kata::plan_unspread(cp);
    CHECK(un.sp == 0 && 2 * (un.states_bytes / 256) >= cp.states_bytes / 256 &&
              un.ws_bytes == un.states_bytes + un.scan_ws_bytes,
          "unspread plan");
  }
  CHECK(u128(cp.states_bytes) ==
            round256(u128(cp.n_seq) * u128(cp.n_seg) * u128(cp.sp ? 2 : 1) *
                     u128(cp.state_elems) * 4),
        "states bytes are the exact product");
  CHECK(cp.states_bytes % 256 == 0, "states aligned");
  CHECK(u128(cp.ws_bytes) == u128(cp.states_bytes) + u128(cp.scan_ws_bytes), "workspace sum");
  if (!cp.walk_sums_prefix)
    CHECK(cp.scan_ws_bytes == kata::plan_scan(cp.n_seq, cp.n_seg, cp.state_elems).ws_bytes,
          "scan workspace");
  check_scan(cp.n_seq, cp.n_seg, cp.state_elems);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: plan_fuzz <seed> <iterations>\n");
    return 2;
  }
  g_state = std::strtoull(argv[1], nullptr, 10);
  const long iters = std::strtol(argv[2], nullptr, 10);
  long valid[3] = {0, 0, 0};
  for (long it = 0; it < iters; ++it) {
    const kata_problem pr = draw();
    g_pr = &pr;
    const kata::Form forms[3] = {kata::Form::Quadratic, kata::Form::Chunked, kata::Form::Backward};
    for (int f = 0; f < 3; ++f) {
      std::string why;
      const kata_status s = kata::validate_problem(&pr, forms[f], &why);
      CHECK(s >= KATA_OK && s <= KATA_ERR_DEVICE, "status code");
      CHECK((s == KATA_OK) == why.empty(), "message exactly on error");
      CHECK(kata::validate_problem(&pr, forms[f], nullptr) == s, "same status without a message");
      if (s != KATA_OK) continue;
      ++valid[f];
      CHECK(pr.B >= 1 && pr.H >= 1 && pr.T >= 1 && pr.T <= kata::kMaxT, "sizes within caps");
      CHECK(int64_t(pr.B) * pr.H <= 65535, "B * H within cap");
      CHECK(pr.p == 8 || pr.p == 16 || pr.p == 32, "p");
      CHECK(pr.dv == 16 || pr.dv == 64, "dv");
      CHECK(std::isfinite(pr.eps) && pr.eps >= 0.f, "eps");
      CHECK(kata::dtype_pair_ok(pr.in_dtype, pr.out_dtype, forms[f]), "dtype pair");
      const int64_t* st[5] = {pr.sq, pr.sk, pr.sv, pr.so, pr.sdo};
      const int64_t last[5] = {pr.p, pr.p, pr.dv, pr.dv, pr.dv};
      for (int i = 0; i < (forms[f] == kata::Form::Backward ? 5 : 4); ++i) {
        for (int a = 0; a < 3; ++a) CHECK(st[i][a] >= 0, "accepted strides are nonnegative");
        CHECK(extent_bytes(pr, st[i], last[i], 4) < (i128(1) << 62), "extent below 2^62 bytes");
      }
      for (int i = 0; i < 4; ++i) {
        const size_t es = kata::elem_size(i < 3 ? pr.in_dtype : pr.out_dtype);
        std::string w2;
        const kata_status t = kata::validate_tensor(reinterpret_cast<const void*>(uintptr_t(1) << 40),
                                                    st[i], es, "x", &w2);
        CHECK(t == KATA_OK || t == KATA_ERR_INVALID_ARGUMENT, "tensor status");
        if (t == KATA_OK)
          for (int a = 0; a < 3; ++a) CHECK(u128(st[i][a]) * es % 16 == 0, "16-byte rows");
      }
      if (forms[f] == kata::Form::Chunked) {
        CHECK(pr.chunk == 16 || pr.chunk == 32 || pr.chunk == 64, "chunk");
        CHECK(pr.T % pr.chunk == 0, "T % chunk");
        check_chunked(pr, true);
        check_chunked(pr, false);
      }
      if (forms[f] == kata::Form::Backward)
        CHECK(u128(kata::bwd_workspace_bytes(&pr)) ==
                  2 * round256(u128(pr.B) * u128(pr.H) * u128(pr.T) * 4),
              "backward workspace");
    }
    // null pointers and misaligned bases are rejected whatever the problem
    std::string w3;
    CHECK(kata::validate_problem(nullptr, kata::Form::Chunked, &w3) == KATA_ERR_INVALID_ARGUMENT,
          "null problem");
    CHECK(kata::validate_tensor(nullptr, pr.sq, 2, "q", &w3) == KATA_ERR_INVALID_ARGUMENT, "null q");
    CHECK(kata::validate_tensor(reinterpret_cast<const void*>(uintptr_t(8)), pr.sq, 2, "q", &w3) ==
              KATA_ERR_INVALID_ARGUMENT,
          "misaligned q");
    // stand-alone scans: the same checks for every size validate_scan accepts
    {
      const int64_t ns = pick<int64_t>({1, 16, 65535, 65536, 0, -1}), n = size_value();
      const int64_t el = pick<int64_t>({4, 10496, 66560, 70000 * 4, int64_t(1) << 30, 6, 0});
      std::string w4;
      const kata_status s = kata::validate_scan(ns, n, el, &w4);
      CHECK(s == KATA_OK || s == KATA_ERR_INVALID_ARGUMENT, "scan status");
      CHECK((s == KATA_OK) == w4.empty(), "scan message exactly on error");
      if (s == KATA_OK) {
        CHECK(u128(ns) * u128(n) * u128(el) * 4 < (u128(1) << 62), "accepted scan below 2^62 bytes");
        check_scan(ns, n, el);
      }
    }
  }
  std::printf("ok %ld problems; valid quadratic %ld, chunked %ld, backward %ld\n", iters,
              valid[0], valid[1], valid[2]);
  return 0;
}

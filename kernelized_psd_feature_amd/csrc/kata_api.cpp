// Host implementation of the C ABI declared in include/kata.h.
//
// Every entry point validates its arguments on the host (plan.cpp), checks that the current
// device is a gfx950, then enqueues its kernels on the caller's stream and returns without
// synchronizing.  Scratch memory comes from the caller's workspace, except for
// kata_fwd_chunked_noalloc, which uses the static per-device array defined below.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "device.h"
#include "kata.h"
#include "plan.h"

namespace kata {
hipError_t launch_quadratic_mfma(const DevProblem& pr, int gw, bool out_bf16, const void* q,
                                 const void* k, const void* v, void* o, float* den,
                                 hipStream_t st);
bool quadratic_mfma_grid_fits(const DevProblem& pr);
int quadratic_mfma_group_width(const kata_problem* pr);
bool chunk_fast_available();
hipError_t launch_chunk_state32(const DevProblem& pr, int L, int n_seg, int n_used, int sp,
                                const void* k, const void* v, float* states, hipStream_t st);
hipError_t launch_chunk_output32(const DevProblem& pr, bool out_bf16, int L, int n_seg, int sp,
                                 const void* q, const void* k, const void* v, void* o,
                                 float* den, const float* states, bool sum_prefix, hipStream_t st);

// Segment states; segments seg >= n_used get a zero state without reading their tokens.
hipError_t launch_chunk_state_fast(const DevProblem& pr, bool packed, int gw, int L, int n_seg,
                                   int n_used, const void* k, const void* v, float* states,
                                   hipStream_t st);
hipError_t launch_halves_combine(const DevProblem& pr, bool out_bf16, const float* o0,
                                 const float* d0, const float* o1, const float* d1, void* o,
                                 float* den, hipStream_t st);
hipError_t launch_chunk_output_fast(const DevProblem& pr, bool packed, int gw, bool out_bf16,
                                    int L, int n_seg, const void* q, const void* k,
                                    const void* v, void* o, float* den, const float* states,
                                    bool sum_prefix, hipStream_t st);
}  // namespace kata

namespace {

using kata::Form;

thread_local std::string g_last_error;

kata_status set_error(kata_status s, const std::string& why) {
  g_last_error = why;
  return s;
}

// ---- device check: the code objects in this library are built for gfx950 only ----------
constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
int g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

kata_status check_device(void) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(KATA_ERR_DEVICE, std::string("no usable HIP device: ") +
                                          hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_dev_mutex);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return set_error(KATA_ERR_DEVICE, std::string("hipGetDeviceProperties failed: ") +
                                            hipGetErrorString(e));
    g_dev_state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    if (g_dev_state[dev] < 0) g_last_error = std::string("device is ") + prop.gcnArchName;
  }
  if (g_dev_state[dev] < 0) return set_error(KATA_ERR_DEVICE, "device is not a gfx950");
  return KATA_OK;
}

// ---- optional per-kernel timing ----------------------------------------------------
struct TimingRec {
  int kind;
  hipEvent_t a, b;
};
struct TimingState {
  bool on = false;
  std::vector<TimingRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local TimingState g_timing;

// The open timing scope of this host thread: the launches inside it (kata::launch_kernel)
// stamp its events with their own dispatch timestamps.
thread_local kata::LaunchTiming* g_scope = nullptr;

// One timing record per scope when timing is on: the span from the start of the scope's first
// kernel to the end of its last (no record if it launched nothing).
struct Timed {
  int kind;
  kata::LaunchTiming lt;
  kata::LaunchTiming* prev = nullptr;
  bool open = false;
  Timed(int kind_, hipStream_t) : kind(kind_) {
    if (!g_timing.on) return;
    lt.start = g_timing.get();
    lt.stop = g_timing.get();
    if (lt.start && lt.stop) {
      prev = g_scope;
      g_scope = &lt;
      open = true;
    } else {
      if (lt.start) g_timing.pool.push_back(lt.start);
      if (lt.stop) g_timing.pool.push_back(lt.stop);
      lt.start = lt.stop = nullptr;
    }
  }
  ~Timed() {
    if (!open) return;
    g_scope = prev;
    if (lt.used) {
      g_timing.recs.push_back({kind, lt.start, lt.stop});
    } else {
      g_timing.pool.push_back(lt.start);
      g_timing.pool.push_back(lt.stop);
    }
  }
  Timed(const Timed&) = delete;
  Timed& operator=(const Timed&) = delete;
};

}  // namespace

namespace kata {
LaunchTiming* launch_timing() { return g_scope; }

hipError_t ensure_dynamic_lds(const void* kernel, int bytes) {
  struct Entry {
    const void* kernel;
    int dev, bytes;
  };
  static std::mutex m;
  static std::vector<Entry> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(m);
  for (const Entry& x : done)
    if (x.kernel == kernel && x.dev == dev && x.bytes >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.push_back({kernel, dev, bytes});
  return e;
}
}  // namespace kata

namespace {

kata::DevProblem to_dev(const kata_problem* pr) {
  kata::DevProblem d;
  d.B = pr->B;
  d.H = pr->H;
  d.T = pr->T;
  d.p = pr->p;
  d.dv = pr->dv;
  d.C = pr->chunk;
  d.gs = pr->groups > 1 ? pr->p / pr->groups : pr->p;
  d.stored_compact = 0;
  d.eps = pr->eps;
  for (int i = 0; i < 3; ++i) {
    d.sq[i] = pr->sq[i];
    d.sk[i] = pr->sk[i];
    d.sv[i] = pr->sv[i];
    d.so[i] = pr->so[i];
    d.sdo[i] = pr->sdo[i];
  }
  return d;
}

kata_status launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KATA_OK;
  return set_error(KATA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

kata_status check_forward_args(const kata_problem* pr, Form f, const void* q, const void* k,
                               const void* v, const void* o, const float* den) {
  std::string why;
  kata_status s = kata::validate_problem(pr, f, &why);
  if (s != KATA_OK) return set_error(s, why);
  const size_t ei = kata::elem_size(pr->in_dtype), eo = kata::elem_size(pr->out_dtype);
  if ((s = kata::validate_tensor(q, pr->sq, ei, "q", &why)) != KATA_OK) return set_error(s, why);
  if ((s = kata::validate_tensor(k, pr->sk, ei, "k", &why)) != KATA_OK) return set_error(s, why);
  if ((s = kata::validate_tensor(v, pr->sv, ei, "v", &why)) != KATA_OK) return set_error(s, why);
  if ((s = kata::validate_tensor(o, pr->so, eo, "o", &why)) != KATA_OK) return set_error(s, why);
  if (den && reinterpret_cast<uintptr_t>(den) % 4)
    return set_error(KATA_ERR_INVALID_ARGUMENT, "den is not 4-byte aligned");
  return KATA_OK;
}

// Recursive prefix scan driver (see plan_scan).
hipError_t run_scan(float* x, int64_t n_seq, int64_t n, int64_t elems, int exclusive,
                    float* totals, char* ws, hipStream_t st) {
  kata::ScanPlan sp = kata::plan_scan(n_seq, n, elems);
  if (sp.wave) return kata::launch_scan_short(x, n_seq, n, elems, exclusive, totals, st);
  if (sp.n_tiles == 1)
    return kata::launch_scan_tiles(x, n_seq, n, elems, (int)sp.strip, (int)n, 1, exclusive,
                                   totals, nullptr, st);
  float* sums = reinterpret_cast<float*>(ws);
  char* sub = ws + ((size_t(n_seq) * sp.n_tiles * elems * 4 + 255) & ~size_t(255));
  hipError_t e = kata::launch_tile_sums(x, n_seq, n, elems, (int)sp.tile_rows,
                                        (int)sp.n_tiles, sums, st);
  if (e != hipSuccess) return e;
  e = run_scan(sums, n_seq, sp.n_tiles, elems, 1, nullptr, sub, st);
  if (e != hipSuccess) return e;
  return kata::launch_scan_tiles(x, n_seq, n, elems, (int)sp.strip, (int)sp.tile_rows,
                                 (int)sp.n_tiles, exclusive, totals, sums, st);
}

// The chunked pipeline for one problem and its plan: segment states, their prefix (scan or
// summed in the walks), the walk; or the fp32 kernels.  Arguments already validated.
kata_status run_chunked(const kata_problem* pr, const kata::ChunkPlan& cp, const void* q,
                        const void* k, const void* v, void* o, float* den, void* workspace,
                        hipStream_t st) {
  kata::DevProblem dp = to_dev(pr);
  dp.stored_compact = cp.compact;
  const bool in_bf16 = pr->in_dtype == KATA_BF16, out_bf16 = pr->out_dtype == KATA_BF16;
  float* states = reinterpret_cast<float*>(workspace);
  char* scan_ws = reinterpret_cast<char*>(workspace) + cp.states_bytes;
  hipError_t e;
  // One segment per sequence (the sequential inter-chunk form): every walk starts from a zero
  // prefix, so no segment state or scan is needed.
  const bool one_segment = cp.fast && cp.n_seg == 1;
  if (!one_segment) {
    {
      Timed t(KATA_K_CHUNK_STATE, st);
      // the last segment's state enters no prefix
      e = cp.fast32 ? kata::launch_chunk_state32(dp, cp.L, cp.n_seg, cp.n_seg - 1, cp.sp, k, v,
                                                 states, st)
          : cp.fast ? kata::launch_chunk_state_fast(dp, cp.packed, cp.gw, cp.L, cp.n_seg,
                                                    cp.n_seg - 1, k, v, states, st)
                    : kata::launch_chunk_state_generic(dp, in_bf16, k, v, states, cp.n_chunks, st);
    }
    if (e != hipSuccess) return launch_status(e, "chunk-state kernel");
    if (!cp.walk_sums_prefix) {
      // exclusive prefix over segments
      Timed t(KATA_K_SCAN, st);
      e = run_scan(states, cp.n_seq, cp.n_seg, cp.state_elems, 1, nullptr, scan_ws, st);
    }
    if (e != hipSuccess) return launch_status(e, "chunk-state scan");
  }
  {
    Timed t(KATA_K_CHUNK_OUTPUT, st);
    const float* pre = one_segment ? nullptr : states;
    const bool sum_prefix = cp.walk_sums_prefix != 0;
    e = cp.fast32 ? kata::launch_chunk_output32(dp, out_bf16, cp.L, cp.n_seg, cp.sp, q, k, v, o,
                                                den, pre, sum_prefix, st)
        : cp.fast ? kata::launch_chunk_output_fast(dp, cp.packed, cp.gw, out_bf16, cp.L,
                                                   cp.n_seg, q, k, v, o, den, pre, sum_prefix, st)
                : kata::launch_chunk_output_generic(dp, in_bf16, out_bf16, q, k, v, o, den,
                                                    states, cp.n_chunks, st);
  }
  return launch_status(e, "chunk-output kernel");
}

// The chunked forward after validation (both entry points): the pipeline of run_chunked, or
// for p = 32 KATA-Mg its two p = 16 passes and their combination.
kata_status chunked_forward(const kata_problem* pr, const kata::ChunkPlan& cp, const void* q,
                            const void* k, const void* v, void* o, float* den, void* workspace,
                            hipStream_t st);

// ---- static scratch of kata_fwd_chunked_noalloc --------------------------------------
// One array per device (each device that loads the library holds its own copy until the
// process ends).  Host code never uses the array's name as an address: the device address is
// taken once per device with hipGetSymbolAddress, with that device current, and kept.
static __device__ __align__(256) unsigned char scratch[KATA_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

kata_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(KATA_ERR_DEVICE, std::string("no usable HIP device: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return set_error(KATA_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch) failed: ") +
                                            hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KATA_OK;
}

}  // namespace

extern "C" {

const char* kata_status_string(kata_status s) {
  switch (s) {
    case KATA_OK: return "ok";
    case KATA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KATA_ERR_UNSUPPORTED: return "unsupported problem";
    case KATA_ERR_WORKSPACE: return "workspace missing or too small";
    case KATA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* kata_last_error(void) { return g_last_error.c_str(); }

kata_status kata_fwd_quadratic(const kata_problem* pr, const void* q, const void* k,
                               const void* v, void* o, float* den, void* stream) {
  g_last_error.clear();
  kata_status s = check_forward_args(pr, Form::Quadratic, q, k, v, o, den);
  if (s != KATA_OK) return s;
  if ((s = check_device()) != KATA_OK) return s;
  const kata::DevProblem dp = to_dev(pr);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool in_bf16 = pr->in_dtype == KATA_BF16, out_bf16 = pr->out_dtype == KATA_BF16;
  const int gw = kata::quadratic_mfma_group_width(pr);   // 0: the fp32 kernel
  if (gw && !kata::quadratic_mfma_grid_fits(dp))
    return set_error(KATA_ERR_UNSUPPORTED, "quadratic forward: more than 2^31 - 1 query blocks");
  Timed t(KATA_K_QUADRATIC, st);
  if (gw)
    return launch_status(kata::launch_quadratic_mfma(dp, gw, out_bf16, q, k, v, o, den, st),
                         "quadratic forward");
  return launch_status(kata::launch_quadratic_generic(dp, in_bf16, out_bf16, q, k, v, o, den, st),
                       "quadratic forward");
}

size_t kata_fwd_chunked_workspace_size(const kata_problem* pr) {
  if (kata::validate_problem(pr, Form::Chunked, nullptr) != KATA_OK) return 0;
  return kata::plan_chunked(pr, kata::chunk_fast_available()).ws_bytes;
}

kata_status kata_fwd_chunked_plan(const kata_problem* pr, kata_chunked_plan* out) {
  g_last_error.clear();
  if (!out) return set_error(KATA_ERR_INVALID_ARGUMENT, "out is null");
  std::string why;
  const kata_status s = kata::validate_problem(pr, Form::Chunked, &why);
  if (s != KATA_OK) return set_error(s, why);
  const kata::ChunkPlan cp = kata::plan_chunked(pr, kata::chunk_fast_available());
  std::memset(out, 0, sizeof(*out));
  out->n_chunks = cp.n_chunks;
  out->chunks_per_segment = cp.L;
  out->segments = cp.n_seg;
  out->state_floats = cp.state_elems;
  out->mfma = cp.fast;
  out->packed = cp.packed;
  out->walk_sums_prefix = cp.walk_sums_prefix;
  const bool no_scan = (cp.fast && cp.n_seg == 1) || cp.walk_sums_prefix;  // as the forward
  out->scan_levels = no_scan ? 0 : kata::plan_scan(cp.n_seq, cp.n_seg, cp.state_elems).levels;
  return KATA_OK;
}

kata_status kata_fwd_chunked(const kata_problem* pr, const void* q, const void* k,
                             const void* v, void* o, float* den, void* workspace,
                             size_t ws_bytes, void* stream) {
  g_last_error.clear();
  kata_status s = check_forward_args(pr, Form::Chunked, q, k, v, o, den);
  if (s != KATA_OK) return s;
  const kata::ChunkPlan cp = kata::plan_chunked(pr, kata::chunk_fast_available());
  if (!workspace || ws_bytes < cp.ws_bytes)
    return set_error(KATA_ERR_WORKSPACE, "workspace needs " + std::to_string(cp.ws_bytes) +
                                             " bytes, got " + std::to_string(ws_bytes));
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return set_error(KATA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if ((s = check_device()) != KATA_OK) return s;
  return chunked_forward(pr, cp, q, k, v, o, den, workspace, reinterpret_cast<hipStream_t>(stream));
}

kata_status kata_fwd_chunked_noalloc(const kata_problem* pr, const void* q, const void* k,
                                     const void* v, void* o, float* den, void* stream) {
  g_last_error.clear();
  kata_status s = check_forward_args(pr, Form::Chunked, q, k, v, o, den);
  if (s != KATA_OK) return s;
  kata::ChunkPlan cp = kata::plan_chunked(pr, kata::chunk_fast_available());
  if (cp.ws_bytes > KATA_NOALLOC_SCRATCH_BYTES) cp = kata::plan_unspread(cp);
  if (cp.ws_bytes > KATA_NOALLOC_SCRATCH_BYTES)
    return set_error(KATA_ERR_WORKSPACE,
                     "the problem needs " + std::to_string(cp.ws_bytes) +
                         " bytes of scratch; the library's static scratch holds " +
                         std::to_string(size_t(KATA_NOALLOC_SCRATCH_BYTES)) +
                         " (use kata_fwd_chunked with a workspace)");
  if ((s = check_device()) != KATA_OK) return s;
  void* ws = nullptr;
  if ((s = static_scratch(&ws)) != KATA_OK) return s;
  return chunked_forward(pr, cp, q, k, v, o, den, ws, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {
kata_status chunked_forward(const kata_problem* pr, const kata::ChunkPlan& cp, const void* q,
                            const void* k, const void* v, void* o, float* den, void* workspace,
                            hipStream_t st) {
  kata_status s;
  if (!cp.halves) return run_chunked(pr, cp, q, k, v, o, den, workspace, st);
  // p = 32 KATA-Mg: two p = 16 passes over the coordinate halves (each with g / 2 groups) into
  // fp32 temporaries, then o = (o_0 D_0 + o_1 D_1) / (D_0 + D_1 - eps)
  char* ws = reinterpret_cast<char*>(workspace);
  const size_t pass_ws = cp.ws_bytes - 2 * (cp.half_out_bytes + cp.half_den_bytes);
  float* oj[2] = {reinterpret_cast<float*>(ws + pass_ws),
                  reinterpret_cast<float*>(ws + pass_ws + cp.half_out_bytes)};
  float* dj[2] = {reinterpret_cast<float*>(ws + pass_ws + 2 * cp.half_out_bytes),
                  reinterpret_cast<float*>(ws + pass_ws + 2 * cp.half_out_bytes +
                                           cp.half_den_bytes)};
  for (int j = 0; j < 2; ++j) {
    kata_problem half = *pr;
    half.p = 16;
    half.groups = (pr->groups <= 1 ? 1 : pr->groups) / 2;
    half.out_dtype = KATA_F32;
    half.so[2] = pr->dv;
    half.so[1] = int64_t(pr->H) * pr->dv;
    half.so[0] = int64_t(pr->T) * half.so[1];
    const __bf16* qh = static_cast<const __bf16*>(q) + 16 * j;   // coordinates 16j .. 16j + 15
    const __bf16* kh = static_cast<const __bf16*>(k) + 16 * j;
    if ((s = run_chunked(&half, cp, qh, kh, v, oj[j], dj[j], workspace, st)) != KATA_OK)
      return s;
  }
  Timed t(KATA_K_CHUNK_OUTPUT, st);
  return launch_status(kata::launch_halves_combine(to_dev(pr), pr->out_dtype == KATA_BF16,
                                                   oj[0], dj[0], oj[1], dj[1], o, den, st),
                       "two-pass combine");
}
}  // namespace

extern "C" {

size_t kata_chunk_state_scan_workspace_size(int64_t n_seq, int64_t n_chunks,
                                            int64_t state_elems) {
  if (kata::validate_scan(n_seq, n_chunks, state_elems, nullptr) != KATA_OK) return 0;
  return kata::plan_scan(n_seq, n_chunks, state_elems).ws_bytes;
}

kata_status kata_chunk_state_scan(float* states, int64_t n_seq, int64_t n_chunks,
                                  int64_t state_elems, int32_t exclusive, float* totals,
                                  void* workspace, size_t ws_bytes, int32_t* levels,
                                  void* stream) {
  g_last_error.clear();
  if (!states) return set_error(KATA_ERR_INVALID_ARGUMENT, "states is null");
  std::string why;
  if (kata::validate_scan(n_seq, n_chunks, state_elems, &why) != KATA_OK)
    return set_error(KATA_ERR_INVALID_ARGUMENT, why);
  if (reinterpret_cast<uintptr_t>(states) % 16 || (totals && reinterpret_cast<uintptr_t>(totals) % 16))
    return set_error(KATA_ERR_INVALID_ARGUMENT, "states/totals must be 16-byte aligned");
  const kata::ScanPlan sp = kata::plan_scan(n_seq, n_chunks, state_elems);
  if (sp.ws_bytes && (!workspace || ws_bytes < sp.ws_bytes))
    return set_error(KATA_ERR_WORKSPACE, "workspace needs " + std::to_string(sp.ws_bytes) +
                                             " bytes, got " + std::to_string(ws_bytes));
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 256)
    return set_error(KATA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if (levels) *levels = sp.levels;
  kata_status s = check_device();
  if (s != KATA_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Timed t(KATA_K_SCAN, st);
  return launch_status(run_scan(states, n_seq, n_chunks, state_elems, exclusive ? 1 : 0,
                                totals, reinterpret_cast<char*>(workspace), st),
                       "chunk-state scan");
}

namespace {
// The recurrent-state build always uses the direct layout: its result is the public
// [dv + 1][p^2] state, which the sum kernel writes from direct segment states.
static kata::ChunkPlan recurrent_plan(const kata_problem* pr) {
  kata_problem d = *pr;
  d.state_layout = KATA_STATE_DIRECT;
  kata::ChunkPlan cp = kata::plan_chunked(&d, kata::chunk_fast_available());
  // the public state is the direct one: p = 32 and KATA-Mg prefill on the fp32 state kernel
  if (cp.fast32 || cp.gw != 16 || cp.halves) cp = kata::plan_chunked(&d, false);
  return cp;
}

static kata_status check_state(const float* state) {
  if (!state) return set_error(KATA_ERR_INVALID_ARGUMENT, "state is null");
  if (reinterpret_cast<uintptr_t>(state) % 16)
    return set_error(KATA_ERR_INVALID_ARGUMENT, "state is not 16-byte aligned");
  return KATA_OK;
}
}  // namespace

size_t kata_recurrent_state_workspace_size(const kata_problem* pr) {
  if (kata::validate_problem(pr, Form::Chunked, nullptr) != KATA_OK) return 0;
  return recurrent_plan(pr).states_bytes;
}

kata_status kata_recurrent_state(const kata_problem* pr, const void* k, const void* v,
                                 float* state, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  std::string why;
  kata_status s = kata::validate_problem(pr, Form::Chunked, &why);
  if (s != KATA_OK) return set_error(s, why);
  const size_t ei = kata::elem_size(pr->in_dtype);
  if ((s = kata::validate_tensor(k, pr->sk, ei, "k", &why)) != KATA_OK) return set_error(s, why);
  if ((s = kata::validate_tensor(v, pr->sv, ei, "v", &why)) != KATA_OK) return set_error(s, why);
  if ((s = check_state(state)) != KATA_OK) return s;
  const kata::ChunkPlan cp = recurrent_plan(pr);
  if (!workspace || ws_bytes < cp.states_bytes)
    return set_error(KATA_ERR_WORKSPACE, "workspace needs " + std::to_string(cp.states_bytes) +
                                             " bytes, got " + std::to_string(ws_bytes));
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return set_error(KATA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if ((s = check_device()) != KATA_OK) return s;
  const kata::DevProblem dp = to_dev(pr);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* states = reinterpret_cast<float*>(workspace);
  hipError_t e;
  {
    Timed t(KATA_K_CHUNK_STATE, st);
    e = cp.fast ? kata::launch_chunk_state_fast(dp, false, 16, cp.L, cp.n_seg, cp.n_seg, k, v,
                                                states, st)
                : kata::launch_chunk_state_generic(dp, pr->in_dtype == KATA_BF16, k, v, states,
                                                   cp.n_chunks, st);
  }
  if (e != hipSuccess) return launch_status(e, "chunk-state kernel");
  Timed t(KATA_K_STATE_SUM, st);
  return launch_status(kata::launch_state_sum(states, cp.n_seq, cp.n_seg, cp.state_elems,
                                              cp.fast != 0, state, st),
                       "state sum");
}

kata_status kata_decode(const kata_problem* pr, const void* q, const void* k, const void* v,
                        void* o, float* den, float* state, void* stream) {
  g_last_error.clear();
  kata_status s = check_forward_args(pr, Form::Quadratic, q, k, v, o, den);
  if (s != KATA_OK) return s;
  if ((s = check_state(state)) != KATA_OK) return s;
  if ((s = check_device()) != KATA_OK) return s;
  const kata::DevProblem dp = to_dev(pr);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Timed t(KATA_K_DECODE, st);
  return launch_status(kata::launch_decode(dp, pr->in_dtype == KATA_BF16,
                                           pr->out_dtype == KATA_BF16, q, k, v, o, den, state,
                                           st),
                       "decode");
}

size_t kata_bwd_workspace_size(const kata_problem* pr) {
  if (kata::validate_problem(pr, Form::Backward, nullptr) != KATA_OK) return 0;
  return kata::bwd_workspace_bytes(pr);
}

kata_status kata_bwd(const kata_problem* pr, const void* q, const void* k, const void* v,
                     const void* dO, void* dq, void* dk, void* dv, void* workspace,
                     size_t ws_bytes, void* stream) {
  g_last_error.clear();
  std::string why;
  kata_status s = kata::validate_problem(pr, Form::Backward, &why);
  if (s != KATA_OK) return set_error(s, why);
  const size_t ei = kata::elem_size(pr->in_dtype);
  struct {
    const void* p;
    const int64_t* st;
    size_t es;
    const char* name;
  } ts[] = {{q, pr->sq, ei, "q"},  {k, pr->sk, ei, "k"},  {v, pr->sv, ei, "v"},
            {dO, pr->sdo, ei, "dO"}, {dq, pr->sq, 4, "dq"}, {dk, pr->sk, 4, "dk"},
            {dv, pr->sv, 4, "dv"}};
  for (auto& x : ts)
    if ((s = kata::validate_tensor(x.p, x.st, x.es, x.name, &why)) != KATA_OK)
      return set_error(s, why);
  const size_t need = kata::bwd_workspace_bytes(pr);
  if (!workspace || ws_bytes < need)
    return set_error(KATA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) +
                                             " bytes, got " + std::to_string(ws_bytes));
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return set_error(KATA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if ((s = check_device()) != KATA_OK) return s;
  const kata::DevProblem dp = to_dev(pr);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool in_bf16 = pr->in_dtype == KATA_BF16;
  float* D = reinterpret_cast<float*>(workspace);
  float* delta = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + need / 2);
  Timed t(KATA_K_BWD, st);
  hipError_t e = kata::launch_bwd_prep(dp, in_bf16, q, k, v, dO, D, delta, st);
  if (e == hipSuccess)
    e = kata::launch_bwd_dq(dp, in_bf16, q, k, v, dO, D, delta, static_cast<float*>(dq), st);
  if (e == hipSuccess)
    e = kata::launch_bwd_dkdv(dp, in_bf16, q, k, v, dO, D, delta, static_cast<float*>(dk),
                              static_cast<float*>(dv), st);
  return launch_status(e, "backward");
}

namespace {
struct BwdChunkedLayout {
  int64_t n_seq = 0, n_chunks = 0, elems = 0;
  size_t states = 0, scan = 0, g = 0, e = 0, total = 0;
};

static BwdChunkedLayout bwd_chunked_layout(const kata_problem* pr) {
  auto r256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  BwdChunkedLayout L;
  L.n_seq = int64_t(pr->B) * pr->H;
  L.n_chunks = pr->T / pr->chunk;
  L.elems = int64_t(pr->p) * pr->p * (pr->dv + 1);
  const size_t tokens = size_t(pr->B) * pr->T * pr->H;
  L.states = r256(size_t(L.n_seq) * L.n_chunks * L.elems * 4);
  L.scan = r256(kata::plan_scan(L.n_seq, L.n_chunks, L.elems).ws_bytes);
  L.g = r256(tokens * pr->dv * 4);
  L.e = r256(tokens * 4);
  L.total = L.states + L.scan + L.g + L.e;
  return L;
}
}  // namespace

size_t kata_bwd_chunked_workspace_size(const kata_problem* pr) {
  if (kata::validate_problem(pr, Form::Chunked, nullptr) != KATA_OK) return 0;
  return bwd_chunked_layout(pr).total;
}

kata_status kata_bwd_chunked(const kata_problem* pr, const void* q, const void* k,
                             const void* v, const void* dO, void* dq, void* dk, void* dv,
                             void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  std::string why;
  kata_status s = kata::validate_problem(pr, Form::Chunked, &why);
  if (s != KATA_OK) return set_error(s, why);
  const size_t ei = kata::elem_size(pr->in_dtype);
  struct {
    const void* p;
    const int64_t* st;
    size_t es;
    const char* name;
  } ts[] = {{q, pr->sq, ei, "q"},  {k, pr->sk, ei, "k"},  {v, pr->sv, ei, "v"},
            {dO, pr->sdo, ei, "dO"}, {dq, pr->sq, 4, "dq"}, {dk, pr->sk, 4, "dk"},
            {dv, pr->sv, 4, "dv"}};
  for (auto& x : ts)
    if ((s = kata::validate_tensor(x.p, x.st, x.es, x.name, &why)) != KATA_OK)
      return set_error(s, why);
  const BwdChunkedLayout L = bwd_chunked_layout(pr);
  if (!workspace || ws_bytes < L.total)
    return set_error(KATA_ERR_WORKSPACE, "workspace needs " + std::to_string(L.total) +
                                             " bytes, got " + std::to_string(ws_bytes));
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return set_error(KATA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if ((s = check_device()) != KATA_OK) return s;
  kata::DevProblem dp = to_dev(pr);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool in_bf16 = pr->in_dtype == KATA_BF16;
  char* ws = reinterpret_cast<char*>(workspace);
  float* states = reinterpret_cast<float*>(ws);
  char* scan_ws = ws + L.states;
  float* g = reinterpret_cast<float*>(ws + L.states + L.scan);
  float* e = reinterpret_cast<float*>(ws + L.states + L.scan + L.g);
  const int nc = int(L.n_chunks);
  // fp32 forward: o (into g) and D_t (into e), leaving the exclusive prefix states
  kata::DevProblem dpo = dp;
  dpo.so[0] = int64_t(pr->T) * pr->H * pr->dv;
  dpo.so[1] = int64_t(pr->H) * pr->dv;
  dpo.so[2] = pr->dv;
  Timed t(KATA_K_BWD, st);
  hipError_t err = kata::launch_chunk_state_generic(dp, in_bf16, k, v, states, nc, st);
  if (err == hipSuccess)
    err = run_scan(states, L.n_seq, L.n_chunks, L.elems, 1, nullptr, scan_ws, st);
  if (err == hipSuccess)
    err = kata::launch_chunk_output_generic(dpo, in_bf16, false, q, k, v, g, e, states, nc, st);
  if (err == hipSuccess) err = kata::launch_bwd_chunk_prep(dp, in_bf16, dO, g, e, st);
  if (err == hipSuccess)
    err = kata::launch_bwd_chunk_dq(dp, in_bf16, q, k, v, g, e, states, nc,
                                    static_cast<float*>(dq), st);
  // reverse chunk states of the queries, suffix sums by the same exclusive scan
  if (err == hipSuccess) err = kata::launch_bwd_rev_state(dp, in_bf16, q, g, e, states, nc, st);
  if (err == hipSuccess)
    err = run_scan(states, L.n_seq, L.n_chunks, L.elems, 1, nullptr, scan_ws, st);
  if (err == hipSuccess)
    err = kata::launch_bwd_chunk_dkdv(dp, in_bf16, q, k, v, g, e, states, nc,
                                      static_cast<float*>(dk), static_cast<float*>(dv), st);
  return launch_status(err, "chunked backward");
}

kata_status kata_timing_begin(void) {
  g_last_error.clear();
  for (auto& r : g_timing.recs) {
    g_timing.pool.push_back(r.a);
    g_timing.pool.push_back(r.b);
  }
  g_timing.recs.clear();
  g_timing.on = true;
  return KATA_OK;
}

kata_status kata_timing_end(kata_kernel_times* out) {
  g_last_error.clear();
  if (!out) return set_error(KATA_ERR_INVALID_ARGUMENT, "out is null");
  if (!g_timing.on) return set_error(KATA_ERR_INVALID_ARGUMENT, "timing was not begun");
  g_timing.on = false;
  std::memset(out, 0, sizeof(*out));
  kata_status s = KATA_OK;
  for (auto& r : g_timing.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      s = set_error(KATA_ERR_DEVICE, "event timing failed");
    if (r.kind >= 0 && r.kind < KATA_K_COUNT) {
      out->launches[r.kind] += 1;
      out->total_ms[r.kind] += ms;
    }
    g_timing.pool.push_back(r.a);
    g_timing.pool.push_back(r.b);
  }
  g_timing.recs.clear();
  return s;
}

}  // extern "C"

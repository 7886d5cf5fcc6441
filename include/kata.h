/*
 * kata.h -- C ABI of the MI355X (gfx950) library for causal, normalized linear attention
 * with the rank-one PSD feature map psi(u) = u u^T ("KATA").
 *
 * What every forward call computes, per batch b and head h, for t = 0 .. T-1:
 *
 *     o_t = sum_{s<=t} (q_t . k_s)^2 v_s  /  (eps + sum_{s<=t} (q_t . k_s)^2)
 *
 * Sources: gist.science "Technische Samenvatting", section 2.2 (psi(u) = u u^T squares the raw
 * inner product) and section 2.1 (the normalizing denominator is a convex output gate);
 * ai.info "AI summary", Main Findings, the bullet on the free readout gate.  eps is added once,
 * outside the sum; the diagonal s = t is included; q and k are used as given (no scaling).
 *
 * Conventions shared by every call
 *   - All data pointers are DEVICE pointers on the current HIP device, owned by the caller.
 *     The library never allocates, frees or retains them; scratch memory comes only from the
 *     caller's workspace, whose size is queried first (kata_fwd_chunked_noalloc alone uses a
 *     static array inside the library instead).  Inputs are read-only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns without synchronizing.  A kernel fault shows
 *     up at the caller's next synchronization, not in the return code.
 *   - Tensor layout: q, k are [B][T][H][p], v and o are [B][T][H][d_v] (the layout of the
 *     pages' kernel call, KATA README), addressed through ELEMENT strides for the (b, t, h)
 *     axes; the last axis is contiguous.  Head-major [B][H][T][D] is the same call with other
 *     strides.  Every row (the base pointer and each stride times the element size) must be
 *     16-byte aligned.
 *   - Validation happens on the host, before anything is enqueued: a call that returns an
 *     error has launched nothing.  No call aborts or throws across the ABI.
 *   - Thread safety: calls may come from several host threads; the only global state is a
 *     lazily filled per-device property cache and the optional timing recorder (one per
 *     host thread).
 */
#ifndef KATA_H
#define KATA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KATA_OK = 0,
  KATA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, stride, alignment or eps       */
  KATA_ERR_UNSUPPORTED = 2,      /* a valid problem the library has no kernel for         */
  KATA_ERR_WORKSPACE = 3,        /* workspace pointer null or smaller than required       */
  KATA_ERR_DEVICE = 4            /* no usable gfx950 device, or a launch error            */
} kata_status;

typedef enum { KATA_F32 = 0, KATA_BF16 = 1 } kata_dtype;

/* Storage of the chunk states S = sum vec(k k^T) v^T of the chunked form.  S is symmetric in
 * its (i, j) feature pair (vec(k k^T) is), so its p(p+1)/2 unique rows determine it exactly
 * (ai.info AI summary, Main Findings, state-size bullet: d^2 outer-product entries or
 * d(d+1)/2 unique packed coordinates).  DIRECT keeps all p^2 rows; PACKED keeps the unique
 * rows with the off-diagonal ones counted twice, so phi(q)^T S is read out over half the rows.
 * Both give the same outputs up to rounding. */
typedef enum { KATA_STATE_DIRECT = 0, KATA_STATE_PACKED = 1 } kata_state_layout;

/* One attention problem.  Sizes:
 *   B, H, T >= 1;  p in {8, 16, 32} (q/k width);  dv in {16, 64} (value width);
 *   chunk: C for the chunked form, one of {16, 32, 64}, T % C == 0 (ignored by the quadratic
 *          form); chunk c covers tokens [cC, (c+1)C).
 *   seg_chunks: chunked form only: chunks per segment L (0 = library default).  The chunked
 *          form keeps the running state on chip for L consecutive chunks and combines the
 *          per-segment states with the prefix scan; L = 1 scans every chunk state, and
 *          L >= T / chunk is the sequential inter-chunk form (one segment per sequence carries
 *          the state through every chunk in order; no scan).  The fp32 kernels always scan
 *          every chunk state.
 *   state_layout: chunked form only, a kata_state_layout.  PACKED is implemented by the bf16
 *          p = 16, dv = 64, chunk = 64 kernels; the bf16 p = 32 ones and the bf16 p = 16
 *          KATA-Mg ones always pack; every other problem computes the direct form whatever
 *          this field says.
 *   groups: KATA-Mg factor count g (0 or 1: the single PSD factor above).  The p coordinates
 *          form g groups of p/g consecutive entries and the score becomes
 *          a_ts = sum_j (q_t^(j) . k_s^(j))^2, with the same single denominator (gist.science
 *          section 2.3, the variants bullet; ai.info Main Findings, state-size bullet; the KATA
 *          README's concat-SPD call with num_groups).  g must divide p.  The bf16 MFMA
 *          kernels (dv = 64; chunk = 64 for the chunked form) take g = 2 and 4 at p = 16 and
 *          keep only the within-group feature pairs; at p = 32 the quadratic form takes
 *          g = 2, 4, 8 on MFMA, and the chunked form runs them as two p = 16 passes over the
 *          coordinate halves (g / 2 groups each) whose numerators and denominators are added
 *          (workspace for the two passes' fp32 outputs included); every other grouped
 *          problem runs the fp32 kernels, whose chunk states keep p^2 rows, the pairs across
 *          groups being zero.
 *   eps: finite, >= 0 (1e-6 in every workload).
 *   in_dtype: dtype of q, k, v (and dO); out_dtype: dtype of o.  Allowed pairs:
 *          (BF16 -> F32), (BF16 -> BF16), (F32 -> F32).  Gradients are always F32.
 *   sq, sk, sv, so, sdo: element strides of the (b, t, h) axes of q, k, v, o and dO.
 *          Gradient outputs dq, dk, dv use the strides of q, k, v respectively. */
typedef struct {
  int32_t B, H, T, p, dv;
  int32_t chunk;
  int32_t seg_chunks;
  int32_t state_layout;
  int32_t groups;
  float eps;
  int32_t in_dtype;
  int32_t out_dtype;
  int64_t sq[3], sk[3], sv[3], so[3], sdo[3];
} kata_problem;

/* Flash-style O(T^2) forward: tiles of Q K^T, squared and causally masked, then P V and a
 * row sum for the denominator; the feature state is never formed.
 * Source: gist.science section 2.3 (quadratic operating point, FlashAttention-style kernel
 * that does not materialize the state); KATA README (direct kernel call on (B,T,H,D)).
 *   q, k, v: inputs as above.  o: output [B][T][H][dv] of out_dtype.
 *   den: optional (NULL allowed) fp32 [B][T][H], contiguous, receives D_t = eps + sum_s a.
 * Errors: INVALID_ARGUMENT / UNSUPPORTED / DEVICE as described above. */
kata_status kata_fwd_quadratic(const kata_problem* pr, const void* q, const void* k,
                               const void* v, void* o, float* den, void* stream);

/* Bytes of device workspace kata_fwd_chunked needs for this problem (0 for an invalid one). */
size_t kata_fwd_chunked_workspace_size(const kata_problem* pr);

/* Exact O(T) chunked-state forward.  For each chunk c the state is
 *     dS_c = sum_{s in c} vec(k_s k_s^T) v_s^T  (p^2 x dv),   dZ_c = sum_{s in c} k_s k_s^T,
 * an exclusive prefix scan gives S_{<c}, Z_{<c}, and for t in chunk c
 *     o_t = (vec(q_t q_t^T)^T S_{<c} + sum_{s in c, s<=t} a_ts v_s)
 *           / (eps + q_t^T Z_{<c} q_t + sum_{s in c, s<=t} a_ts).
 * Source: gist.science section 2.3 (chunked parallelism: intra-chunk attention on matrix
 * units, inter-chunk state propagation by an associative scan, depth O(log N_C)); ai.info
 * Main Findings (chunk recurrence without a triangular solve; state size); the paper review's
 * Validation paragraph (the chunked-state form is exact).
 * Arguments as kata_fwd_quadratic, plus a device workspace of at least
 * kata_fwd_chunked_workspace_size(pr) bytes, 256-byte aligned; its contents on entry are
 * ignored and on exit undefined.  Errors: as above, plus WORKSPACE. */
kata_status kata_fwd_chunked(const kata_problem* pr, const void* q, const void* k,
                             const void* v, void* o, float* den, void* workspace,
                             size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): kata_fwd_chunked without a workspace.  The segment
 * states and the scan's scratch live in a static array inside the library, one per device,
 * KATA_NOALLOC_SCRATCH_BYTES long, held from the library's first use on that device until the
 * process ends; the call itself allocates nothing (no hipMalloc, no allocating library call).
 * Arguments, results and errors are those of kata_fwd_chunked (same kernels, same plan, the
 * same outputs bit for bit), except:
 *   - a problem whose kata_fwd_chunked_workspace_size exceeds KATA_NOALLOC_SCRATCH_BYTES is
 *     rejected with KATA_ERR_WORKSPACE before anything is enqueued (the 131072-token, 16-head
 *     p = 16 plan needs 30.8 MiB; the literal one-state-per-chunk scan there, 1.3 GiB, does
 *     not fit) -- unless its p = 32 state pass is spread (see kata_chunked_plan) and one state
 *     per segment, half those states' bytes, fits: then it runs that way, and its outputs
 *     agree with kata_fwd_chunked's to rounding (the prefixes add the same chunks in another
 *     grouping) rather than bit for bit;
 *   - every call on one device shares that device's array and leaves its contents behind
 *     (nothing in it has to start at zero): calls that may overlap in time on one device --
 *     on different streams, or from different host threads -- race and must be ordered by
 *     the caller (e.g. one stream). */
#define KATA_NOALLOC_SCRATCH_BYTES (64u << 20)
kata_status kata_fwd_chunked_noalloc(const kata_problem* pr, const void* q, const void* k,
                                     const void* v, void* o, float* den, void* stream);

/* The plan kata_fwd_chunked takes for a problem (host only; no device call).  The chunks of
 * one (b, h) are walked in `segments` segments of `chunks_per_segment` chunks; a state pass
 * and an exclusive prefix scan over the segment states, a combining tree of `scan_levels`
 * levels, feed the walk.  With one segment per (b, h) on the MFMA kernels (the sequential
 * inter-chunk form) neither runs and scan_levels is 0.  With 2 to 8 segments on the MFMA
 * kernels (walk_sums_prefix = 1) no scan runs either (scan_levels 0): the walk of segment s adds
 * the states of segments 0 .. s-1 in that order, the same exclusive prefix (p = 32 with at most
 * 4 segments: the state pass spreads those chunks over one workgroup per segment, and the walk
 * adds the sums of the ranges before its first chunk in chunk order, the range that crosses it
 * up to that chunk; state_floats is still the size of one state).  For p = 32
 * KATA-Mg on the MFMA kernels the plan is that of each of the two p = 16 passes.  Source:
 * gist.science section 2.3 (inter-chunk depth O(log N_C)).
 *   out: host struct, filled on success.
 * Errors: INVALID_ARGUMENT (NULL out, or as kata_fwd_chunked), UNSUPPORTED. */
typedef struct {
  int64_t n_chunks;            /* T / chunk, per (b, h) */
  int64_t chunks_per_segment;
  int64_t segments;            /* per (b, h) */
  int64_t state_floats;        /* fp32 values in one segment state */
  int32_t scan_levels;
  int32_t mfma;                /* 1: bf16 MFMA kernels; 0: fp32 kernels */
  int32_t packed;              /* 1: states keep only the unique (i <= j) feature pairs */
  int32_t walk_sums_prefix;    /* 1: the walks add the earlier segment states, no scan */
} kata_chunked_plan;
kata_status kata_fwd_chunked_plan(const kata_problem* pr, kata_chunked_plan* out);

/* Bytes of workspace kata_chunk_state_scan needs (0 when n_chunks fits one tree). */
size_t kata_chunk_state_scan_workspace_size(int64_t n_seq, int64_t n_chunks,
                                            int64_t state_elems);

/* Associative prefix scan over chunk states, in place, fp32:
 *     states[s][c][e]  <-  sum_{i<c} states[s][i][e]    (exclusive != 0)
 *     states[s][c][e]  <-  sum_{i<=c} states[s][i][e]   (exclusive == 0)
 * for every sequence s < n_seq and element e < state_elems, each element independently.
 * The operator is plain addition because the state update is additive and commutative
 * (ai.info Main Findings, readout-gate bullet); it is evaluated as a Kogge-Stone tree of depth
 * ceil(log2 n_chunks) (gist.science section 2.3: depth O(N_C) -> O(log N_C); the paper
 * review's Results paragraph: O(log(T/C))).
 *   states: device fp32 [n_seq][n_chunks][state_elems], contiguous, 16-byte aligned,
 *           state_elems % 4 == 0.
 *   totals: optional device fp32 [n_seq][state_elems]: receives the inclusive total (the
 *           state after the last chunk).
 *   workspace/ws_bytes: at least kata_chunk_state_scan_workspace_size(...) bytes (NULL/0 when
 *           that is 0).
 *   levels: optional host int32 out: the depth of the combining tree that was run.
 * Errors: INVALID_ARGUMENT, WORKSPACE, DEVICE. */
kata_status kata_chunk_state_scan(float* states, int64_t n_seq, int64_t n_chunks,
                                  int64_t state_elems, int32_t exclusive, float* totals,
                                  void* workspace, size_t ws_bytes, int32_t* levels,
                                  void* stream);

/* ---- Recurrent form: prefill and decode ---------------------------------------------
 * The state of one (b, h) after tokens 0 .. t is
 *     S_t = sum_{s<=t} vec(k_s k_s^T) v_s^T  (p^2 x dv),   Z_t = sum_{s<=t} k_s k_s^T,
 * and o_t = vec(q_t q_t^T)^T S_t / (eps + q_t^T Z_t q_t): the same outputs as the forms above,
 * computed with a constant-size state per token (ai.info AI summary, Main Findings, the bullet
 * on constant-time recurrent inference; gist.science section 2.2 for vec(u u^T)).
 * State layout: device fp32 [B][H][dv + 1][p * p], contiguous, 16-byte aligned; row d < dv of
 * a (b, h) holds S[(i, j)][d] at column i * p + j, row dv holds Z[i][j] at column i * p + j.
 */

/* Bytes of workspace kata_recurrent_state needs (0 for an invalid problem). */
size_t kata_recurrent_state_workspace_size(const kata_problem* pr);

/* Prefill: state <- (S, Z) after the problem's T tokens, from k and v (q is not read).  The
 * problem is checked as for kata_fwd_chunked (T % chunk == 0; state_layout is ignored); the
 * bf16 p = 16, dv = 64, chunk = 64, g = 1 problem uses the MFMA state kernel (phi(k) rounded to
 * bf16 before the products with v, fp32 accumulation), every other one fp32 arithmetic.  The state
 * is overwritten.  Errors: as kata_fwd_chunked. */
kata_status kata_recurrent_state(const kata_problem* pr, const void* k, const void* v,
                                 float* state, void* workspace, size_t ws_bytes, void* stream);

/* Decode: advances state over the problem's T tokens one at a time (T = 1 is one decode step)
 * and writes o_t (and D_t = eps + q_t^T Z_t q_t into den if not NULL) for each, all
 * arithmetic in fp32.  pr->chunk, seg_chunks and state_layout are ignored.  state is read and
 * written in place; calls that share a state must be ordered on one stream.
 * Errors: INVALID_ARGUMENT / UNSUPPORTED / DEVICE as for the forward calls. */
kata_status kata_decode(const kata_problem* pr, const void* q, const void* k, const void* v,
                        void* o, float* den, float* state, void* stream);

/* Bytes of workspace kata_bwd needs. */
size_t kata_bwd_workspace_size(const kata_problem* pr);

/* Gradients of L = sum_t <dO_t, o_t> with respect to q, k, v, all arithmetic in fp32:
 *     delta_t = dO_t . o_t,   G_ts = (dO_t . v_s - delta_t) / D_t   (s <= t)
 *     dq_t = sum_s 2 (q_t.k_s) G_ts k_s,  dk_s = sum_t 2 (q_t.k_s) G_ts q_t,
 *     dv_s = sum_{t>=s} (q_t.k_s)^2 dO_t / D_t.
 * Source: the KATA README names a flash forward/backward; the formulas are the derivative
 * of the closed form above (the pages print none).
 *   dO: [B][T][H][dv] of in_dtype (strides sdo).  dq, dk, dv: fp32 outputs with the strides
 *   of q, k, v.  The workspace holds D_t and delta_t (fp32 [B][T][H] each).
 * Errors: as kata_fwd_chunked. */
kata_status kata_bwd(const kata_problem* pr, const void* q, const void* k, const void* v,
                     const void* dO, void* dq, void* dk, void* dv, void* workspace,
                     size_t ws_bytes, void* stream);

/* Bytes of workspace kata_bwd_chunked needs (0 for an invalid problem). */
size_t kata_bwd_chunked_workspace_size(const kata_problem* pr);

/* The same gradients as kata_bwd in O(T): the chunked forward's exclusive prefix states give
 * the part of dq from earlier chunks,
 *     dq_t += 2 [mat(S_{<c} g_t) - e_t Z_{<c}] q_t,   g_t = dO_t / D_t, e_t = delta_t / D_t,
 * and a suffix scan over chunks of R = sum vec(q q^T) g^T and r = sum e vec(q q^T) (the
 * prefix scan run over the chunk states stored in reverse order) gives the part of dk and dv
 * from later chunks,
 *     dk_s += 2 [mat(R_{>c} v_s) - mat(r_{>c})] k_s,   dv_s += R_{>c}^T vec(k_s k_s^T);
 * the terms inside a chunk are its causal tile.  Source: derived from the chunked form of
 * gist.science section 2.3 (states, associative scan) and the closed form above; the pages
 * print no backward.  All arithmetic is fp32 (the forward pass inside included).
 * Arguments as kata_bwd; the problem is checked as for kata_fwd_chunked (T % chunk == 0).
 * The workspace holds one fp32 state of p^2 (dv + 1) floats per chunk and (b, h), the scan's
 * workspace, and g_t, e_t.  Errors: as kata_bwd. */
kata_status kata_bwd_chunked(const kata_problem* pr, const void* q, const void* k,
                             const void* v, const void* dO, void* dq, void* dk, void* dv,
                             void* workspace, size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* kata_status_string(kata_status s);

/* Text describing the last error returned on this host thread ("" if none). */
const char* kata_last_error(void);

/* ---- Per-kernel timing (measurement support; off by default) --------------------------
 * kata_timing_begin(): on this host thread, from now on every kernel kind an entry point runs
 * is timed by a pair of HIP events that its kernels' own dispatches stamp (launched with
 * hipExtLaunchKernel on the caller's stream, so no marker packets sit between kernels): the
 * span from the start of its first kernel to the end of its last.
 * kata_timing_end(): synchronizes those events and returns, per kernel kind, the number of
 * launches and the summed elapsed milliseconds; recording stops.  Kinds are indexed by
 * kata_kernel_kind.  Returns INVALID_ARGUMENT if begin was not called, DEVICE on an event
 * error. */
typedef enum {
  KATA_K_QUADRATIC = 0,
  KATA_K_CHUNK_STATE = 1,
  KATA_K_SCAN = 2,
  KATA_K_CHUNK_OUTPUT = 3,
  KATA_K_BWD = 4,
  KATA_K_DECODE = 5,
  KATA_K_STATE_SUM = 6,
  KATA_K_COUNT = 7
} kata_kernel_kind;

typedef struct {
  int64_t launches[KATA_K_COUNT];
  double total_ms[KATA_K_COUNT];
} kata_kernel_times;

kata_status kata_timing_begin(void);
kata_status kata_timing_end(kata_kernel_times* out);

#ifdef __cplusplus
}
#endif

#endif /* KATA_H */

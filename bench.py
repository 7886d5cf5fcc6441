"""Throughput benchmark of the chunked-state forward (the hot path), one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_context_131k]

A step is one kata_fwd_chunked call (segment-state build, prefix scan over the segment
states -- formed inside the walk instead when a sequence has at most 8 segments --, intra-chunk
tiles + inter-chunk readout + output gate) over the whole workload, with q, k, v already
resident in HBM and the output and workspace preallocated.  W untimed steps, then K
steps timed with HIP events on the stream the kernels are launched on (value, ms_per_step),
then K more steps in which the library's own per-kernel events on the same stream give the
dominant kernel's average duration for the roofline figure (those events add a few
microseconds per kernel, so that pass's step time is reported separately).

Printed: one JSON line.  value = head-tokens (B*H*T) per second.  roofline: the algorithmic
bytes (bf16 q, k, v in, fp32 o out) or flops of the step, whichever bound is slower at MI355X's
peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16 MFMA), over the dominant kernel's average duration.
step_roofline: the same for the whole step (every kernel of it).  warmup_steps_run: the untimed
steps actually run before the timed ones (at least W, more until --warmup-floor-s seconds of
load have passed).  literal_scan: the 131k workload with one state per chunk and the 11-level
prefix scan over them.
cpu_baseline: the fp64 CPU oracle (brute-force closed form) timed on a bounded uniform sample
of the same workload's query rows, scaled to head-tokens/s.  sweep: tokens/s of the chunked
form at T = 1k .. 128k with B*T = 131072 (the metric's dependence on T), each beside the
sequential inter-chunk form (one segment per sequence, no scan), the ratio of the two, and the
quadratic form.  crossover (--workload crossover_p32): both forms at p = 32, T = 1k .. 16k.

    python bench.py --form decode     # one decode step for 512 x 16 heads (recurrent form)
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd tokens/sec (B·H·T/s) at p=16,d_v=64 vs T; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
KERNEL_SOURCES = {  # files whose content defines each kernel's code
    "chunk_output": ["kernelized_psd_feature_amd/csrc/fast.hip",
                     "kernelized_psd_feature_amd/csrc/mfma_util.h",
                     "kernelized_psd_feature_amd/csrc/device.h"],
    "quadratic": ["kernelized_psd_feature_amd/csrc/quadratic.hip",
                  "kernelized_psd_feature_amd/csrc/mfma_util.h",
                  "kernelized_psd_feature_amd/csrc/device.h"],
    "decode": ["kernelized_psd_feature_amd/csrc/decode.hip",
               "kernelized_psd_feature_amd/csrc/device.h"],
    "chunk_output32": ["kernelized_psd_feature_amd/csrc/fast32.hip",
                       "kernelized_psd_feature_amd/csrc/mfma_util.h",
                       "kernelized_psd_feature_amd/csrc/device.h"],
    "quadratic32": ["kernelized_psd_feature_amd/csrc/quadratic.hip",
                    "kernelized_psd_feature_amd/csrc/mfma_util.h",
                    "kernelized_psd_feature_amd/csrc/device.h"],
}


def algorithmic_bytes_per_token(p, dv, in_bytes=2, out_bytes=4):
    # read q, k (p each) and v (dv) once, write o (dv) once
    return in_bytes * (2 * p + dv) + out_bytes * dv


def chunked_flops_per_token(p, dv, C, groups=1):
    # with n = p^2 / g state features (g KATA-Mg groups of p / g coordinates; n = p^2 at g = 1):
    # state build and readout 2 n (d_v + 1) each, intra-chunk tile (C+1)/2 causal pairs on
    # average of 2 (p + d_v + 1) (score, PV, row sum), q^T Z q 2 n, the scan's
    # 2 n (d_v + 1) / C, epilogue d_v
    n = p * p // groups
    return (4 * n * (dv + 1) + (C + 1) * (p + dv + 1) + 2 * n + 2 * n * (dv + 1) // C + dv)


def quadratic_flops_per_token(p, dv, T):
    # (T + 1) / 2 causal pairs per query on average, 2 (p + d_v + 1) flops each, epilogue d_v
    return (T + 1) * (p + dv + 1) + dv


def roofline(flops, nbytes, seconds):
    """The bound is whichever of the MFMA (bf16 dense) and HBM rooflines takes longer for
    the algorithmic flops and bytes; achieved = that quantity / the measured time."""
    t_mfma = flops / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if t_mfma > t_hbm:
        a = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(a, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a / BF16_MFMA_PEAK_TFLOPS, 4)}
    a = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4)}


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, sha):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the factor a plain device copy of known size
    gives), if the counters were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_sha") != sha:
        return None
    return c.get("traffic_bytes_per_launch")


def cold_cache_ms(step, n, dev):
    """Average step time with the 256 MB Infinity Cache and the L2s flushed before every
    step (a 1 GiB buffer is rewritten outside the timed events)."""
    import torch

    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    total = 0.0
    for _ in range(n):
        flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        total += a.elapsed_time(b)
    del flush
    return total / n


def measured_peaks(dev):
    """The box's own ceilings, for calibration beside the spec peaks (never on the hot path):
    a 1 GiB device-to-device copy (GB/s counting its read and its write) and an 8192^3 bf16
    GEMM through torch (TFLOP/s)."""
    import torch

    stream = torch.cuda.current_stream(dev)

    def seconds(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps / 1e3

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    copy = 2 * n / seconds(lambda: dst.copy_(src), 10) / 1e9
    del src, dst
    m = 8192
    x = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    y = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    gemm = 2 * m ** 3 / seconds(lambda: torch.mm(x, y), 10) / 1e12
    del x, y
    return {"copy_GBps": round(copy, 1), "bf16_gemm_TFLOPs": round(gemm, 1)}


def with_measured_peak(roof, peaks):
    """roofline fraction of the dominant kernel against the box's measured ceiling"""
    ceiling = peaks["copy_GBps"] if roof["bound"] == "hbm" else peaks["bf16_gemm_TFLOPs"]
    return dict(peaks, frac_of_measured=round(roof["achieved"] / ceiling, 4))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_info(dev):
    import torch

    pr = torch.cuda.get_device_properties(dev)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""),
            "compute_units": pr.multi_processor_count, "memory_GiB": round(pr.total_memory / 2**30, 1)}


def input_record(tensors, seed=0):
    """Seed, generator library version and a hash of the exact input bytes (CPU tensors)."""
    import numpy as np
    import torch

    h = hashlib.sha256()
    for x in tensors:
        h.update(x.contiguous().view(-1).view(torch.uint8).numpy().tobytes())
    return {"seed": seed, "numpy": np.__version__, "generator": "kata_workloads.make_inputs",
            "sha256": h.hexdigest()[:16]}


def cpu_baseline(w, target_s=12.0):
    """Time the oracle's closed form on uniformly sampled query rows of one head of the
    workload; head-tokens/s of the oracle on the full workload = rows / seconds (a uniform
    sample has the workload's average cost per row)."""
    import numpy as np
    import torch

    import kata_workloads as W
    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    q, k, v = W.make_inputs(w, 0, B=1, H=1)
    Q, Kk, V = (x[0, :, 0].to(torch.float64).numpy() for x in (q, k, v))
    rng = np.random.default_rng(0)
    n, done, spent = 32, 0, 0.0
    while spent < target_s:
        rows = rng.integers(0, w.T, size=n)
        t0 = time.perf_counter()
        O.closed_form_rows(Q, Kk, V, rows, block=16)
        spent += time.perf_counter() - t0
        done += n
        n = min(4 * n, 4096)
    return {
        "value": done / spent, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{done} query rows drawn uniformly from head 0 (T={w.T}) of the {w.name} "
                  f"workload, fp64 brute-force closed form, {spent:.1f} s",
    }


def warm_up(step, warmup, floor_s=0.0):
    """At least `warmup` untimed steps, and more until `floor_s` seconds of wall time have
    passed (the GPU's clocks take a fraction of a second of load to settle); returns the number
    of steps run.  The host synchronizes every 16 steps, so wall time is GPU time."""
    import torch

    t0, n = time.perf_counter(), 0
    while n < warmup or time.perf_counter() - t0 < floor_s:
        step()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def timed_steps(step, steps, warmup, dev, per_step=False, warmup_floor_s=0.0, info=None):
    """W untimed steps (at least; more until warmup_floor_s seconds have passed, their number
    stored in info["warmup_steps_run"]), then K steps between two events on the launch stream
    (the step time), then K more steps with the library's per-kernel events on the same stream
    (the kernel durations; those events cost a few microseconds per kernel, so they stay out of
    the step time).  Returns (ms per step, {kernel: (launches, total ms)}, instrumented ms per
    step, (median, min) ms of single steps or None): with per_step, K more steps with an event
    after each give the distribution of single-step times."""
    import torch

    import kernelized_psd_feature_amd as K

    n_warm = warm_up(step, warmup, warmup_floor_s)
    if info is not None:
        info["warmup_steps_run"] = n_warm
    stream = torch.cuda.current_stream(dev)

    def region(instrumented):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if instrumented:
            K.timing_begin()
        start.record(stream)
        for _ in range(steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        per_kernel = K.timing_end() if instrumented else None
        return start.elapsed_time(stop) / steps, per_kernel

    ms, _ = region(False)
    ms_inst, per_kernel = region(True)
    dist = None
    if per_step:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        one = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        dist = (one[len(one) // 2], one[0])
    return ms, per_kernel, ms_inst, dist


def graph_ms(step, steps, dev):
    """The step captured once into a HIP graph (torch.cuda.graph records the library's launches
    on its capture stream) and replayed K times between two events: the step time without the
    host's per-call launch costs."""
    import torch

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        g.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def sweep(q, k, v, args, dev):
    """Forward tokens/s of the chunked form at each T of the metric's sweep, B*T = 131072,
    16 heads: the 131k workload's tensors viewed as (131072 / T, T, 16, D); beside it the
    sequential inter-chunk form and the quadratic form on the same tensors."""
    import torch

    import kata_workloads as W
    import kernelized_psd_feature_amd as K

    out = []
    o = torch.empty(v.shape, dtype=torch.float32, device=dev)
    for T in W.SWEEP_T:
        B = q.shape[0] * q.shape[1] // T
        qs, ks, vs, os_ = (x.reshape(B, T, *x.shape[2:]) for x in (q, k, v, o))
        point = {"T": T, "B": B}
        # default segmentation (walks + scan), then the sequential inter-chunk form: one
        # segment per sequence carries the state through all T / 64 chunks
        for key, seg in (("", 0), ("sequential_", T // 64)):
            ws = torch.empty(max(K.chunked_workspace_size(qs, ks, vs, seg_chunks=seg,
                                                          state=args.state), 256),
                             dtype=torch.uint8, device=dev)

            def step():
                K.fwd_chunked(qs, ks, vs, seg_chunks=seg, out=os_, workspace=ws,
                              state=args.state)

            ms, _, _, _ = timed_steps(step, 30, 10, dev)
            point[key + "ms"] = round(ms, 5)
            point[key + "tokens_per_s"] = round(B * 16 * T / (ms / 1e3), 1)
            del ws
        point["scan_speedup"] = round(point["sequential_ms"] / point["ms"], 3)
        # the quadratic form on the same tensors (O(T^2): a few steps at long T)
        ms, _, _, _ = timed_steps(lambda: K.fwd_quadratic(qs, ks, vs, out=os_),
                                  10 if T <= 16384 else 3, 3, dev)
        point["quadratic_ms"] = round(ms, 5)
        point["quadratic_tokens_per_s"] = round(B * 16 * T / (ms / 1e3), 1)
        out.append(point)
    return out


def literal_scan(q, k, v, o, w, args, dev):
    """The chunked form with one state per chunk (seg_chunks = 1): every one of the T / 64 chunk
    states per head is materialized and combined by the prefix scan, ceil(log2(T / 64)) levels
    (11 at T = 131072), as the problem statement writes the inter-chunk step; beside the
    default plan's segment walk it shows what the hierarchical form saves."""
    import torch

    import kernelized_psd_feature_amd as K

    need = K.chunked_workspace_size(q, k, v, chunk=w.chunk, seg_chunks=1, state=args.state)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    plan = K.chunked_plan(q, k, v, chunk=w.chunk, seg_chunks=1, state=args.state)

    def step():
        K.fwd_chunked(q, k, v, chunk=w.chunk, seg_chunks=1, out=o, workspace=ws,
                      state=args.state)

    ms, per_kernel, _, _ = timed_steps(step, 10, 3, dev)
    del ws
    tokens = w.B * w.H * w.T
    return {"ms": round(ms, 5), "tokens_per_s": round(tokens / (ms / 1e3), 1),
            "segments": plan["segments"], "chunks_per_segment": plan["chunks_per_segment"],
            "scan_levels": plan["scan_levels"], "workspace_bytes": need,
            "kernels_ms": {n: round(t / max(c, 1), 5) for n, (c, t) in per_kernel.items() if c}}


def crossover(w, dev):
    """Both forms at each T of the p = 32 crossover workload (B = 4, H = 16, T = 1k .. 16k):
    step times, head-tokens/s and which form is faster there."""
    import torch

    import kata_workloads as W
    import kernelized_psd_feature_amd as K

    out = []
    for T in W.CROSSOVER_T:
        q, k, v = (x.to(dev) for x in W.make_inputs(w, 0, T=T))
        o = torch.empty(v.shape, dtype=torch.float32, device=dev)
        ws = torch.empty(max(K.chunked_workspace_size(q, k, v), 256), dtype=torch.uint8,
                         device=dev)
        point = {"T": T, "B": w.B}
        for form, step in (("chunked", lambda: K.fwd_chunked(q, k, v, out=o, workspace=ws)),
                           ("quadratic", lambda: K.fwd_quadratic(q, k, v, out=o))):
            ms, _, _, _ = timed_steps(step, 20, 20, dev)
            point[form + "_ms"] = round(ms, 5)
            point[form + "_tokens_per_s"] = round(w.B * w.H * T / (ms / 1e3), 1)
        point["faster"] = "chunked" if point["chunked_ms"] < point["quadratic_ms"] else "quadratic"
        out.append(point)
        del q, k, v, o, ws
    return out


def run_chunked(args, dev, w):
    import torch

    import kata_workloads as W
    import kernelized_psd_feature_amd as K

    q, k, v = W.make_inputs(w, 0)
    inputs = input_record((q, k, v))
    if args.layout == "bhtd":
        q, k, v = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    q, k, v = (x.to(dev) for x in (q, k, v))
    out_dtype = torch.bfloat16 if args.out == "bf16" else torch.float32
    o = torch.empty(v.shape, dtype=out_dtype, device=dev)
    ws = None
    if args.form == "chunked":
        need = K.chunked_workspace_size(q, k, v, chunk=w.chunk, seg_chunks=args.seg,
                                        out_dtype=out_dtype, state=args.state,
                                        groups=args.groups)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def step():
        if args.form == "chunked":
            K.fwd_chunked(q, k, v, chunk=w.chunk, seg_chunks=args.seg, out=o, workspace=ws,
                          out_dtype=out_dtype, state=args.state, groups=args.groups)
        else:
            K.fwd_quadratic(q, k, v, out=o, out_dtype=out_dtype, groups=args.groups)

    warm = {}
    ms, per_kernel, ms_inst, dist = timed_steps(step, args.steps, args.warmup, dev, True,
                                                warmup_floor_s=args.warmup_floor_s, info=warm)
    tokens = w.B * w.H * w.T
    dom = "chunk_output" if args.form == "chunked" else "quadratic"
    _, total_ms = per_kernel[dom]
    # the dominant kernel's time per step (one launch per step; at p = 32 with KATA-Mg groups
    # the chunked output stage is two p = 16 walks and their combination)
    avg_ms = total_ms / args.steps
    bpt = algorithmic_bytes_per_token(w.p, w.dv, out_bytes=2 if args.out == "bf16" else 4)
    fpt = (chunked_flops_per_token(w.p, w.dv, w.chunk, args.groups) if args.form == "chunked"
           else quadratic_flops_per_token(w.p, w.dv, w.T))
    sources = KERNEL_SOURCES[dom if w.p == 16 else dom + "32"]
    sha = source_sha(sources)
    roof = roofline(fpt * tokens, bpt * tokens, avg_ms / 1e3)
    # the committed counters were taken with fp32 outputs and one group
    roof["traffic"] = (load_traffic(dom, w.name, sha)
                       if args.out == "fp32" and args.groups == 1 else None)
    line = {
        "metric": METRIC, "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "p": w.p, "dv": w.dv,
                   "chunk": w.chunk, "form": args.form, "seg_chunks": args.seg,
                   "state": args.state, "groups": args.groups, "layout": args.layout.upper(),
                   "out_dtype": args.out, "eps": 1e-6},
        "roofline": roof,
        "kernels_ms": {n: round(t / max(c, 1), 5) for n, (c, t) in per_kernel.items() if c},
        "ms_per_step_with_kernel_events": round(ms_inst, 5),
        "ms_per_step_median": round(dist[0], 5), "ms_per_step_min": round(dist[1], 5),
        "step_roofline": roofline(fpt * tokens, bpt * tokens, ms / 1e3),
        "step_roofline_frac": roofline(fpt * tokens, bpt * tokens, ms / 1e3)["frac"],
        "warmup_floor_s": args.warmup_floor_s, "warmup_steps_run": warm["warmup_steps_run"],
        "dominant_kernel_source_sha": sha,
        "inputs": inputs, "device": device_info(dev),
    }
    if args.form == "chunked":
        line["chunked_plan"] = K.chunked_plan(q, k, v, chunk=w.chunk, seg_chunks=args.seg,
                                              state=args.state, groups=args.groups)
    if args.form == "chunked" and w.name == "long_context_131k" and not args.no_literal \
            and args.layout == "bthd" and args.out == "fp32" and args.groups == 1:
        line["literal_scan"] = literal_scan(q, k, v, o, w, args, dev)
    if args.graph:
        line["ms_per_step_graph"] = round(graph_ms(step, args.steps, dev), 5)
    if not args.no_calibration:
        line["measured_peaks"] = with_measured_peak(roof, measured_peaks(dev))
    if not args.no_cold_cache:
        line["ms_per_step_cold_cache"] = round(cold_cache_ms(step, max(5, args.steps // 5), dev),
                                               5)
    if args.form == "chunked" and w.name == "long_context_131k" and not args.no_sweep \
            and args.layout == "bthd" and args.out == "fp32":
        del ws
        line["sweep"] = sweep(q, k, v, args, dev)
        sp = [x["scan_speedup"] for x in line["sweep"]]
        line["scan_speedup_mean"] = round(sum(sp) / len(sp), 3)
    if args.form == "chunked" and w.name == "crossover_p32" and not args.no_sweep \
            and args.layout == "bthd" and args.out == "fp32" and args.groups == 1:
        line["crossover"] = crossover(w, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    return line


def decode_bytes_per_token(p, dv, in_bytes=2, out_bytes=4):
    # the fp32 state of the (b, h), read once and written once, plus q, k, v in and o out
    return 2 * 4 * p * p * (dv + 1) + algorithmic_bytes_per_token(p, dv, in_bytes, out_bytes)


def cpu_baseline_decode(w, target_s=10.0):
    """Time the oracle's token-by-token recurrence (a decode step per token) on one head of
    the workload's recipe; head-tokens/s."""
    import torch

    import kata_workloads as W
    import oracle as O

    q, k, v = W.make_inputs(w, 0, B=1, H=1, T=64)
    Q, Kk, V = (x.to(torch.float64).numpy() for x in (q, k, v))
    done, spent = 0, 0.0
    while spent < target_s:
        t0 = time.perf_counter()
        O.recurrent(Q, Kk, V)
        spent += time.perf_counter() - t0
        done += Q.shape[1]
    return {"value": done / spent, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} decode steps of one head (p={w.p}, d_v={w.dv}) by the fp64 "
                      f"token-by-token recurrence, {spent:.1f} s"}


def run_decode(args, dev):
    import torch

    import kata_workloads as W
    import kernelized_psd_feature_amd as K

    w = W.DECODE
    cpu = W.make_inputs(w, 0)
    inputs = input_record(cpu)
    q, k, v = (x.to(dev) for x in cpu)
    state = torch.zeros(K.state_shape(k, v), dtype=torch.float32, device=dev)
    o = torch.empty(v.shape, dtype=torch.float32, device=dev)

    def step():
        K.decode(q, k, v, state, out=o)

    warm = {}
    ms, per_kernel, ms_inst, dist = timed_steps(step, args.steps, args.warmup, dev, True,
                                                warmup_floor_s=args.warmup_floor_s, info=warm)
    tokens = w.B * w.H * w.T
    launches, total_ms = per_kernel["decode"]
    avg_ms = total_ms / max(launches, 1)
    bpt = decode_bytes_per_token(w.p, w.dv)
    achieved = bpt * tokens / (avg_ms / 1e3) / 1e9
    line = {
        "metric": "decode tokens/sec (B·H new tokens per step / s), p=16, d_v=64",
        "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "tokens_per_step": w.T, "p": w.p,
                   "dv": w.dv, "form": "decode", "state_bytes": 4 * tokens * w.p ** 2 * (w.dv + 1)},
        "inputs": inputs, "device": device_info(dev),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("decode", w.name,
                                             source_sha(KERNEL_SOURCES["decode"]))},
        "kernels_ms": {n: round(t / max(c, 1), 5) for n, (c, t) in per_kernel.items() if c},
        "ms_per_step_with_kernel_events": round(ms_inst, 5),
        "ms_per_step_median": round(dist[0], 5), "ms_per_step_min": round(dist[1], 5),
        "warmup_floor_s": args.warmup_floor_s, "warmup_steps_run": warm["warmup_steps_run"],
    }
    if not args.no_calibration:
        line["measured_peaks"] = with_measured_peak(line["roofline"], measured_peaks(dev))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(w)
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first (at least; see --warmup-floor-s)")
    ap.add_argument("--warmup-floor-s", type=float, default=0.3,
                    help="keep warming up until this much wall time has passed: the clocks "
                         "need a fraction of a second of load to settle (the steps run are "
                         "reported as warmup_steps_run)")
    ap.add_argument("--workload", default="long_context_131k")
    ap.add_argument("--form", choices=["chunked", "quadratic", "decode"], default="chunked")
    ap.add_argument("--seg", type=int, default=0, help="chunks per segment (0 = library default)")
    ap.add_argument("--layout", choices=["bthd", "bhtd"], default="bthd")
    ap.add_argument("--state", choices=["direct", "packed"], default="packed",
                    help="chunk-state storage: all p^2 rows or the p(p+1)/2 unique ones")
    ap.add_argument("--groups", type=int, default=1,
                    help="KATA-Mg factor count g (1: the single PSD factor)")
    ap.add_argument("--out", choices=["fp32", "bf16"], default="fp32",
                    help="output dtype: fp32 (parity mode, the headline) or bf16 (fast mode)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a HIP graph (ms_per_step_graph)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the T sweep")
    ap.add_argument("--no-literal", action="store_true",
                    help="skip the one-state-per-chunk (literal scan) form")
    ap.add_argument("--no-cold-cache", action="store_true",
                    help="skip the cache-flushed repetition (profiler runs)")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the measured copy and GEMM ceilings")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="run only a device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(every (batch, head) is independent; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import kata_workloads as W

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}), flush=True)
        return
    if args.form == "decode":
        line = run_decode(args, dev)
    else:
        w = next(x for x in W.WORKLOADS.values() if x.name == args.workload)
        line = run_chunked(args, dev, w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

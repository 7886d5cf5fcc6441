"""bench.py's host-side arithmetic and contract, on the CPU: the algorithmic byte and flop
counts per head-token, the roofline bound selection, the committed traffic lookup and the
one-GPU exit."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bytes_per_head_token():
    # bf16 q, k (p each) and v (d_v) in, fp32 o (d_v) out
    assert bench.algorithmic_bytes_per_token(16, 64) == 2 * (16 + 16 + 64) + 4 * 64 == 448
    assert bench.algorithmic_bytes_per_token(16, 64, out_bytes=2) == 320
    assert bench.algorithmic_bytes_per_token(32, 64) == 512
    # decode: the fp32 state p^2 (d_v + 1) read and written, plus the token's own I/O
    assert bench.decode_bytes_per_token(16, 64) == 2 * 4 * 256 * 65 + 448 == 133568


def test_flops_per_head_token():
    # chunked: 4 p^2 (d_v + 1) + (C + 1)(p + d_v + 1) + 2 p^2 + 2 p^2 (d_v + 1) / C + d_v
    assert bench.chunked_flops_per_token(16, 64, 64) == 66560 + 5265 + 512 + 520 + 64 == 72921
    assert bench.chunked_flops_per_token(32, 64, 64) == 276737
    # KATA-Mg: g groups keep n = p^2 / g features (g = 2 at p = 16: 128)
    n = 128
    assert bench.chunked_flops_per_token(16, 64, 64, groups=2) == \
        4 * n * 65 + 65 * 81 + 2 * n + 2 * n * 65 // 64 + 64
    # quadratic: (T + 1)(p + d_v + 1) + d_v
    assert bench.quadratic_flops_per_token(16, 64, 2048) == 2049 * 81 + 64 == 166033


def test_roofline_takes_the_slower_bound():
    # 1 GB and 1e11 flop: HBM takes 125 us, MFMA 40 us -> HBM-bound
    r = bench.roofline(1e11, 1e9, 250e-6)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert r["achieved"] == pytest.approx(4000.0) and r["frac"] == pytest.approx(0.5)
    # 1 PFLOP and 1 GB: MFMA-bound
    r = bench.roofline(1e15, 1e9, 1.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(1000.0 / bench.BF16_MFMA_PEAK_TFLOPS, rel=1e-3)
    # the 131k-token chunked step is HBM-bound (arithmetic intensity 163 flop/B < the ridge)
    tok = 16 * 131072
    r = bench.roofline(bench.chunked_flops_per_token(16, 64, 64) * tok,
                       bench.algorithmic_bytes_per_token(16, 64) * tok, 1e-3)
    assert r["bound"] == "hbm"


def test_committed_traffic_is_reported_only_for_the_source_it_was_taken_on():
    # the walk's counters under profiles/ name the source sha they were taken on; bench.py
    # reports their traffic only while the kernel source still has that sha (else null)
    with open(os.path.join(ROOT, "profiles", "chunk_output_long_context_131k_counters.json")) as f:
        c = json.load(f)
    assert c["kernel_sources"] == bench.KERNEL_SOURCES["chunk_output"]
    traffic = bench.load_traffic("chunk_output", "long_context_131k", c["kernel_source_sha"])
    assert traffic == c["traffic_bytes_per_launch"]
    alg = bench.algorithmic_bytes_per_token(16, 64) * 16 * 131072
    assert c["algorithmic_bytes_per_launch"] == alg
    assert alg < traffic < 1.2 * alg
    assert bench.load_traffic("chunk_output", "long_context_131k", "0" * 16) is None
    assert bench.load_traffic("chunk_output", "no_such_workload", c["kernel_source_sha"]) is None


def test_every_profile_summary_names_its_command_and_source():
    pdir = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(pdir))
    assert any(n.endswith("_kernel_trace.md") for n in names)
    for n in names:
        text = open(os.path.join(pdir, n)).read()
        if n.endswith(".md"):
            assert "rocprofv3" in text and "sha" in text, n
        elif n.endswith(".json"):
            c = json.loads(text)
            assert c["kernel_source_sha"] and c["commands"], n


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""

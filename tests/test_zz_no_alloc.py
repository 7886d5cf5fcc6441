"""kata_fwd_chunked_noalloc (the chunked forward on the library's static scratch) against
kata_fwd_chunked with a caller workspace: the same kernels and plan, so the same outputs bit
for bit, on two calls in a row (the second with a smaller input, reusing the scratch the first
left behind), plus the oracle on sampled rows; and a p = 32 problem whose spread state pass
needs more than the scratch, which runs with one state per segment (outputs equal to rounding)."""

import numpy as np
import pytest
import torch

import kata_workloads as W
import kernelized_psd_feature_amd as K
import oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _both(q, k, v, **kw):
    ref, dref = K.fwd_chunked(q, k, v, return_den=True, **kw)
    out = torch.empty_like(ref)
    den = torch.empty_like(dref)
    K.fwd_chunked_noalloc(q, k, v, out, den=den, **kw)
    return ref, dref, out, den


def _oracle_rows(q, k, v, o, heads, rows, groups=1):
    worst = 0.0
    for b, h in heads:
        ref, _ = O.closed_form_rows(q[b, :, h].double().cpu().numpy(),
                                    k[b, :, h].double().cpu().numpy(),
                                    v[b, :, h].double().cpu().numpy(), rows, groups=groups)
        worst = max(worst, float(np.abs(o[b, rows, h].double().cpu().numpy() - ref).max()))
    return worst


def test_noalloc_matches_the_workspace_entry_point_twice_second_smaller():
    # first call: the 131072-token, 16-head workload (its plan needs 30.8 MiB of states);
    # second call: a smaller 340M-layer slice, on the scratch the first call left behind
    w4 = W.WORKLOADS[4]
    q, k, v = (x.to(DEV) for x in W.make_inputs(w4, 0))
    need = K.chunked_workspace_size(q, k, v)
    assert 0 < need <= K.NOALLOC_SCRATCH_BYTES
    ref, dref, out, den = _both(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(den, dref)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(w4.T - 64, w4.T),
                                     np.random.default_rng(5).choice(w4.T, 64, replace=False)]))
    assert _oracle_rows(q, k, v, out, [(0, 0), (0, 15)], rows) <= 1e-2
    del q, k, v, ref, dref, out, den

    w2 = W.WORKLOADS[2]
    q, k, v = (x.to(DEV) for x in W.make_inputs(w2, 1, B=2, H=4, T=1024))
    assert K.chunked_workspace_size(q, k, v) < need
    ref, dref, out, den = _both(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(den, dref)
    assert _oracle_rows(q, k, v, out, [(0, 0), (1, 3)], np.arange(1024)) <= 1e-2


# p32_spread: 4 segments of 10 chunks, the spread p = 32 state pass (two states per segment)
@pytest.mark.parametrize("case", ["p32", "p32_spread", "p16_g2_bf16_out", "p32_g2", "p8_fp32"])
def test_noalloc_other_kernels_match_the_workspace_entry_point(case):
    wid, kw, shape = {"p32": (3, {}, dict(B=2, H=16, T=4096)),
                      "p32_spread": (3, {"seg_chunks": 10}, dict(B=1, H=4, T=2048)),
                      "p16_g2_bf16_out": (2, {"groups": 2}, dict(B=2, H=8, T=2048)),
                      "p32_g2": (3, {"groups": 2}, dict(B=2, H=8, T=2048)),
                      "p8_fp32": (1, {"chunk": 32}, dict(B=2, H=3, T=256))}[case]
    w = W.WORKLOADS[wid]
    q, k, v = (x.to(DEV) for x in W.make_inputs(w, 2, **shape))
    if case == "p16_g2_bf16_out":
        ref = K.fwd_chunked(q, k, v, out_dtype=torch.bfloat16, **kw)
        out = torch.empty_like(ref)
        K.fwd_chunked_noalloc(q, k, v, out, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        return
    ref, dref, out, den = _both(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(den, dref)


def test_noalloc_unspreads_a_p32_state_pass_beyond_its_scratch():
    # p = 32 at 4 x 16 heads x 16384 tokens: 4 segments of 64 chunks; the spread state pass
    # keeps two partial states per segment (73 MB), one state per segment fits (37 MB)
    w = W.WORKLOADS[3]
    q, k, v = (x.to(DEV) for x in W.make_inputs(w, 3, B=4, H=16, T=16384))
    assert K.chunked_workspace_size(q, k, v) > K.NOALLOC_SCRATCH_BYTES
    ref, dref, out, den = _both(q, k, v)
    torch.cuda.synchronize()
    assert float((out - ref).abs().max()) <= 1e-3
    assert float(((den - dref).abs() / dref).max()) <= 1e-4
    rows = np.unique(np.concatenate([np.arange(64), np.arange(4096 - 8, 4096 + 8),
                                     np.arange(16384 - 64, 16384)]))
    assert _oracle_rows(q, k, v, out, [(0, 0), (3, 15)], rows) <= 1e-2


@pytest.mark.parametrize("seg", [3, 5])
def test_noalloc_replays_from_a_hip_graph(seg):
    # what the entry point is for: a forward captured into a HIP graph with nothing allocated.
    # Every replay equals the eager call bitwise, with eager calls of the same entry point on
    # other inputs (the same static scratch) between the replays; seg 3: 11 segments per
    # sequence and the segment scan, seg 5: 7 segments whose walks sum their prefixes
    w = W.WORKLOADS[2]
    q, k, v = (x.to(DEV) for x in W.make_inputs(w, 93, T=2048, B=2, H=4))
    q2, k2, v2 = (x.to(DEV) for x in W.make_inputs(w, 94, T=2048, B=2, H=4))
    plan = K.chunked_plan(q, k, v, seg_chunks=seg)
    assert plan["walk_sums_prefix"] == (seg == 5) and (plan["scan_levels"] > 0) == (seg == 3)
    o = torch.empty(v.shape, dtype=torch.float32, device=DEV)
    eager = K.fwd_chunked_noalloc(q, k, v, torch.empty_like(o), seg_chunks=seg).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        K.fwd_chunked_noalloc(q, k, v, o, seg_chunks=seg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.fwd_chunked_noalloc(q, k, v, o, seg_chunks=seg)
    other = torch.empty_like(o)
    for r in range(4):
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager), f"replay {r} differs from the eager call"
        K.fwd_chunked_noalloc(q2, k2, v2, other, seg_chunks=seg)
        torch.cuda.synchronize()
        assert torch.isfinite(other).all()
    assert torch.equal(eager, K.fwd_chunked(q, k, v, seg_chunks=seg))


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    # one state per chunk (seg_chunks = 1) over 2 x 1024 chunks: 86 MB of states
    w4 = W.WORKLOADS[4]
    q, k, v = (x.to(DEV) for x in W.make_inputs(w4, 0, H=2, T=65536))
    assert K.chunked_workspace_size(q, k, v, seg_chunks=1) > K.NOALLOC_SCRATCH_BYTES
    out = torch.full((1, 65536, 2, 64), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(K.KataError) as e:
        K.fwd_chunked_noalloc(q, k, v, out, seg_chunks=1)
    assert e.value.status == 3 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())                       # nothing was launched

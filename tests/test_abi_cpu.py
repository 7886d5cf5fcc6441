"""C-ABI checks that need no GPU: libkata.so loads, exports every function include/kata.h
declares, and rejects bad arguments with the documented status codes before touching a
device.  Fake (never dereferenced) device pointers are used: validation runs first."""

import ctypes
import math
import os
import re
import shutil
import subprocess

import pytest

import kernelized_psd_feature_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kata.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, DEVICE = 0, 1, 2, 3, 4
FAKE = 0x7F0000000000          # 256-byte aligned, never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = set(re.findall(r"\b(kata_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def _lib():
    if not os.path.exists(K.library_path()):
        pytest.fail("libkata.so is not built (run python -m kernelized_psd_feature_amd.build)")
    return K._lib()


def _problem(B=1, H=2, T=128, p=16, dv=64, chunk=64, eps=1e-6, in_dt=1, out_dt=0, seg=0):
    pr = K._Problem()
    pr.B, pr.H, pr.T, pr.p, pr.dv, pr.chunk, pr.seg_chunks, pr.eps = B, H, T, p, dv, chunk, seg, eps
    pr.in_dtype, pr.out_dtype = in_dt, out_dt
    pr.sq[:] = (T * H * p, H * p, p)
    pr.sk[:] = (T * H * p, H * p, p)
    pr.sv[:] = (T * H * dv, H * dv, dv)
    pr.so[:] = (T * H * dv, H * dv, dv)
    pr.sdo[:] = (T * H * dv, H * dv, dv)
    return pr


def _fake(n=1):
    return [ctypes.c_void_p(FAKE + i * (1 << 30)) for i in range(n)]


def _quad(pr, ptrs=None, den=None):
    q, k, v, o = ptrs or _fake(4)
    return _lib().kata_fwd_quadratic(ctypes.byref(pr) if pr is not None else None, q, k, v, o,
                                     den, None)


def _chunked(pr, ws_bytes=None, ws=True):
    lib = _lib()
    q, k, v, o, w = _fake(5)
    need = lib.kata_fwd_chunked_workspace_size(ctypes.byref(pr))
    return lib.kata_fwd_chunked(ctypes.byref(pr), q, k, v, o, None, w if ws else None,
                                need if ws_bytes is None else ws_bytes, None)


def test_header_declares_the_four_operations():
    names = _declared_functions()
    for f in ("kata_fwd_quadratic", "kata_fwd_chunked", "kata_chunk_state_scan", "kata_bwd"):
        assert f in names


def test_library_exports_every_declared_function():
    lib = _lib()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"


def test_status_strings():
    lib = _lib()
    for s in range(5):
        assert lib.kata_status_string(s)
    assert lib.kata_status_string(99) == b"unknown status"


def test_null_problem_is_invalid():
    assert _quad(None) == INVALID


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, INVALID), ("H", 0, INVALID), ("T", 0, INVALID), ("p", 0, INVALID),
    ("p", 12, UNSUPPORTED), ("p", 64, UNSUPPORTED), ("dv", 32, UNSUPPORTED),
    ("eps", -1.0, INVALID), ("eps", float("nan"), INVALID), ("eps", float("inf"), INVALID),
    ("in_dtype", 7, INVALID), ("out_dtype", 7, INVALID),
    ("groups", -1, INVALID), ("groups", 3, INVALID), ("groups", 17, INVALID),
])
def test_bad_problem_fields(field, value, code):
    pr = _problem()
    setattr(pr, field, value)
    assert _quad(pr) == code
    assert _lib().kata_last_error()


def test_fp32_in_bf16_out_is_rejected():
    assert _quad(_problem(in_dt=0, out_dt=1)) == INVALID


def test_null_and_misaligned_pointers():
    pr = _problem()
    q, k, v, o = _fake(4)
    assert _quad(pr, [None, k, v, o]) == INVALID
    assert _quad(pr, [q, k, v, None]) == INVALID
    assert _quad(pr, [ctypes.c_void_p(FAKE + 2), k, v, o]) == INVALID
    assert _quad(pr, [q, k, v, o], den=ctypes.c_void_p(FAKE + 2)) == INVALID


def test_bad_strides():
    pr = _problem()
    pr.sq[2] = 3                                     # rows overlap
    assert _quad(pr) == INVALID
    pr = _problem()
    pr.sv[1] = pr.sv[1] + 1                          # breaks 16-byte row alignment
    assert _quad(pr) == INVALID
    pr = _problem()
    pr.sk[0] = -1
    assert _quad(pr) == INVALID


def test_chunked_rejects_ragged_T_and_bad_chunk():
    assert _chunked(_problem(T=100)) == UNSUPPORTED
    assert _chunked(_problem(chunk=48)) == UNSUPPORTED
    assert _chunked(_problem(chunk=0)) == INVALID
    assert _chunked(_problem(seg=-1)) == INVALID
    pr = _problem()
    pr.state_layout = 2
    assert _chunked(pr) == INVALID


def test_chunked_workspace_checks():
    pr = _problem()
    need = _lib().kata_fwd_chunked_workspace_size(ctypes.byref(pr))
    assert need > 0
    assert _chunked(pr, ws=False) == WORKSPACE
    assert _chunked(pr, ws_bytes=need - 1) == WORKSPACE


def test_workspace_size_of_invalid_problem_is_zero():
    assert _lib().kata_fwd_chunked_workspace_size(ctypes.byref(_problem(T=100))) == 0
    assert _lib().kata_bwd_workspace_size(ctypes.byref(_problem(p=5))) == 0


def test_packed_state_workspace_holds_the_unique_rows():
    # packed states: the 136 unique rows x 64 (the 24 zero rows of the 10 tiles are not
    # stored) + the 16 x 16 Z, against 256 x 64 + 256 for the direct layout; same
    # segmentation for both
    lib = _lib()
    for T in (1024, 131072):
        d = _problem(B=1, H=16, T=T)
        pk = _problem(B=1, H=16, T=T)
        pk.state_layout = 1
        nd = lib.kata_fwd_chunked_workspace_size(ctypes.byref(d))
        npk = lib.kata_fwd_chunked_workspace_size(ctypes.byref(pk))
        assert 0 < npk < nd
        n_states = 16 * (T // 64) if T == 1024 else None
        if n_states:   # one segment per chunk when the chunks do not fill the GPU
            assert npk >= n_states * (136 * 64 + 256) * 4
            assert nd >= n_states * 16640 * 4
    # a packed request on a problem the MFMA kernels do not take sizes as direct
    f = _problem(B=1, H=2, T=256, p=8, dv=16, chunk=32, in_dt=0)
    fp = _problem(B=1, H=2, T=256, p=8, dv=16, chunk=32, in_dt=0)
    fp.state_layout = 1
    assert lib.kata_fwd_chunked_workspace_size(ctypes.byref(f)) == \
        lib.kata_fwd_chunked_workspace_size(ctypes.byref(fp))


@pytest.mark.parametrize("p,dv", [(8, 16), (16, 64), (32, 64)])
def test_chunked_workspace_holds_the_segment_states(p, dv):
    # one fp32 state of p^2 (dv + 1) entries per segment; at least one segment per (b, h)
    pr = _problem(B=2, H=3, T=256, p=p, dv=dv, chunk=32, in_dt=0)
    need = _lib().kata_fwd_chunked_workspace_size(ctypes.byref(pr))
    assert need >= 2 * 3 * p * p * (dv + 1) * 4


def test_scan_argument_checks():
    lib = _lib()
    (s,) = _fake(1)
    lv = ctypes.c_int32(-1)
    assert lib.kata_chunk_state_scan(None, 1, 4, 16, 1, None, None, 0, None, None) == INVALID
    assert lib.kata_chunk_state_scan(s, 0, 4, 16, 1, None, None, 0, None, None) == INVALID
    assert lib.kata_chunk_state_scan(s, 1, 4, 18, 1, None, None, 0, None, None) == INVALID
    assert lib.kata_chunk_state_scan(ctypes.c_void_p(FAKE + 4), 1, 4, 16, 1, None, None, 0,
                                     None, None) == INVALID
    # hierarchical sizes need a workspace
    need = lib.kata_chunk_state_scan_workspace_size(2, 10000, 64)
    assert need > 0
    assert lib.kata_chunk_state_scan(s, 2, 10000, 64, 1, None, None, 0, ctypes.byref(lv),
                                     None) == WORKSPACE


@pytest.mark.parametrize("n", [1, 2, 3, 8, 64, 100, 2048, 4096])
def test_scan_reports_log_depth(n):
    # a single Kogge-Stone tree: ceil(log2 n) levels (2048 chunk states -> 11)
    lib = _lib()
    assert lib.kata_chunk_state_scan_workspace_size(4, n, 16640) == 0
    lv = ctypes.c_int32(-1)
    st = lib.kata_chunk_state_scan(_fake(1)[0], 4, n, 16640, 1, None, None, 0,
                                   ctypes.byref(lv), None)
    assert lv.value == math.ceil(math.log2(n)) if n > 1 else lv.value == 0
    assert st in (OK, DEVICE)


def test_backward_argument_checks():
    lib = _lib()
    pr = _problem()
    ptrs = _fake(8)
    need = lib.kata_bwd_workspace_size(ctypes.byref(pr))
    assert need >= 2 * 2 * 128 * 4
    args = [ctypes.byref(pr)] + ptrs[:7] + [ptrs[7], need, None]
    bad = list(args)
    bad[4] = None                                     # dO
    assert lib.kata_bwd(*bad) == INVALID
    bad = list(args)
    bad[9] = need - 1
    assert lib.kata_bwd(*bad) == WORKSPACE


def test_valid_call_without_a_gpu_reports_device_error():
    # This container has no GPU: a fully valid call gets past validation and fails cleanly
    # at the device check instead of crashing.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _quad(_problem()) == DEVICE
    assert _lib().kata_last_error()
    lib = _lib()
    q, k, v, o = _fake(4)
    st = ctypes.c_void_p(FAKE + (1 << 24))
    # decode ignores chunk: T = 1 with chunk = 0 passes validation
    one = _problem(T=1, chunk=0)
    assert lib.kata_decode(ctypes.byref(one), q, k, v, o, None, st, None) == DEVICE
    pr = _problem()
    need = lib.kata_recurrent_state_workspace_size(ctypes.byref(pr))
    ws = ctypes.c_void_p(FAKE + (1 << 28))
    assert lib.kata_recurrent_state(ctypes.byref(pr), k, v, st, ws, need, None) == DEVICE


def test_timing_end_without_begin_is_invalid():
    t = K._Times()
    assert _lib().kata_timing_end(ctypes.byref(t)) == INVALID


def test_recurrent_entry_points_check_their_arguments():
    lib = _lib()
    pr = _problem()
    q, k, v, o = _fake(4)
    st = ctypes.c_void_p(FAKE + (1 << 24))
    # decode: null or misaligned state, bad problem
    assert lib.kata_decode(ctypes.byref(pr), q, k, v, o, None, None, None) == INVALID
    assert lib.kata_decode(ctypes.byref(pr), q, k, v, o, None,
                           ctypes.c_void_p(FAKE + 4), None) == INVALID
    bad = _problem(p=12)
    assert lib.kata_decode(ctypes.byref(bad), q, k, v, o, None, st, None) == UNSUPPORTED
    # prefill: checked like the chunked form, plus the state and the workspace
    assert lib.kata_recurrent_state_workspace_size(ctypes.byref(_problem(T=100))) == 0
    need = lib.kata_recurrent_state_workspace_size(ctypes.byref(pr))
    assert need >= 2 * 16 * 16 * 65 * 4
    ws = ctypes.c_void_p(FAKE + (1 << 28))
    assert lib.kata_recurrent_state(ctypes.byref(_problem(T=100)), k, v, st, ws, need, None) == UNSUPPORTED
    assert lib.kata_recurrent_state(ctypes.byref(pr), k, v, None, ws, need, None) == INVALID
    assert lib.kata_recurrent_state(ctypes.byref(pr), k, v, st, ws, need - 1, None) == WORKSPACE
    assert lib.kata_recurrent_state(ctypes.byref(pr), k, v, st, None, need, None) == WORKSPACE
    # the packed request does not change the prefill's (direct) workspace
    pk = _problem()
    pk.state_layout = 1
    assert lib.kata_recurrent_state_workspace_size(ctypes.byref(pk)) == need


def test_chunked_backward_checks_its_arguments():
    lib = _lib()
    pr = _problem()
    t = _fake(7)
    need = lib.kata_bwd_chunked_workspace_size(ctypes.byref(pr))
    # one fp32 state per chunk and (b, h), plus g (dv floats) and e per token
    assert need >= 2 * 2 * 16 * 16 * 65 * 4 + 128 * 2 * 65 * 4
    assert lib.kata_bwd_chunked_workspace_size(ctypes.byref(_problem(T=100))) == 0
    ws = ctypes.c_void_p(FAKE + (1 << 33))
    assert lib.kata_bwd_chunked(ctypes.byref(_problem(T=100)), *t, ws, need, None) == UNSUPPORTED
    assert lib.kata_bwd_chunked(ctypes.byref(pr), *t, ws, need - 1, None) == WORKSPACE
    assert lib.kata_bwd_chunked(ctypes.byref(pr), *t, None, need, None) == WORKSPACE
    t2 = list(t)
    t2[4] = None                                    # dq missing
    assert lib.kata_bwd_chunked(ctypes.byref(pr), *t2, ws, need, None) == INVALID


def test_groups_do_not_change_workspace_sizes():
    # KATA-Mg keeps the p^2-row state layout (pairs across groups are zero rows)
    lib = _lib()
    for g in (0, 1, 2, 4, 16):
        pr = _problem(B=1, H=2, T=256, chunk=32, in_dt=0)
        pr.groups = g
        base = _problem(B=1, H=2, T=256, chunk=32, in_dt=0)
        assert lib.kata_fwd_chunked_workspace_size(ctypes.byref(pr)) == \
            lib.kata_fwd_chunked_workspace_size(ctypes.byref(base))
        assert lib.kata_bwd_chunked_workspace_size(ctypes.byref(pr)) == \
            lib.kata_bwd_chunked_workspace_size(ctypes.byref(base))


def test_p32_spread_state_pass_workspace():
    # with 2 to 4 segments whose walks add the prefixes, the p = 32 state pass keeps two states
    # per segment (the sum of a workgroup's range and of its part before a segment boundary);
    # with more segments one
    lib = _lib()
    out = K._ChunkedPlan()
    state_bytes = (34 * 16 * 64 + 4 * 256) * 4
    for B, H, T, seg, n_seg, per_seg in ((4, 16, 16384, 0, 4, 2), (1, 2, 1024, 7, 3, 2),
                                         (1, 2, 1024, 8, 2, 2), (2, 16, 4096, 0, 8, 1)):
        pr = _problem(B=B, H=H, T=T, p=32, seg=seg)
        assert lib.kata_fwd_chunked_plan(ctypes.byref(pr), ctypes.byref(out)) == OK
        assert (out.segments, out.walk_sums_prefix, out.scan_levels) == (n_seg, 1, 0)
        need = lib.kata_fwd_chunked_workspace_size(ctypes.byref(pr))
        assert need == -(-B * H * n_seg * per_seg * state_bytes // 256) * 256


def test_chunked_plan_reports_segments_and_scan_depth():
    lib = _lib()
    out = K._ChunkedPlan()
    # 131k tokens, 16 heads: segments of several chunks, a prefix scan over them
    pr = _problem(B=1, H=16, T=131072)
    pr.state_layout = 1
    assert lib.kata_fwd_chunked_plan(ctypes.byref(pr), ctypes.byref(out)) == OK
    assert (out.n_chunks, out.mfma, out.packed) == (2048, 1, 1)
    assert out.segments == -(-2048 // out.chunks_per_segment) and 1 < out.segments < 2048
    assert out.scan_levels == math.ceil(math.log2(out.segments)) and out.walk_sums_prefix == 0
    assert out.state_floats == (136 * 64 + 256)           # the 136 unique (i, j) rows x 64, + Z
    # 512 sequences fill two thirds of the GPU's 768 workgroup slots: one segment each, no
    # state pass, no scan; 256 sequences take 3 segments each (768 walks), and with at most 8
    # segments the walks add the earlier segments' states themselves: no scan either
    pr = _problem(B=32, H=16, T=1024)
    assert lib.kata_fwd_chunked_plan(ctypes.byref(pr), ctypes.byref(out)) == OK
    assert (out.segments, out.chunks_per_segment, out.scan_levels) == (1, 16, 0)
    assert out.walk_sums_prefix == 0
    assert out.state_floats == 16 * 16 * 65                # direct layout: p^2 (dv + 1)
    pr = _problem(B=16, H=16, T=8192)
    assert lib.kata_fwd_chunked_plan(ctypes.byref(pr), ctypes.byref(out)) == OK
    assert (out.segments, out.chunks_per_segment, out.scan_levels) == (3, 43, 0)
    assert out.walk_sums_prefix == 1
    # short sequences: the walks' prefix reads decide the segment count.  8 x 16 heads x 2048
    # tokens (32 chunks): 4 segments of 8 (the last walk moves 8 chunks and 3 states) rather
    # than 6 of 6 (6 chunks and 5 states); 8 x 16 x 4096 keeps 6 segments of 11
    for T, n_seg, L in ((2048, 4, 8), (4096, 6, 11)):
        pr = _problem(B=8, H=16, T=T)
        pr.state_layout = 1
        assert lib.kata_fwd_chunked_plan(ctypes.byref(pr), ctypes.byref(out)) == OK
        assert (out.segments, out.chunks_per_segment, out.walk_sums_prefix) == (n_seg, L, 1)
    # p = 32 (MFMA-bound walk, one workgroup per CU) keeps every slot busy: 4 x 16 x 1024
    # stays at 4 segments of 4
    pr = _problem(B=4, H=16, T=1024, p=32)
    assert lib.kata_fwd_chunked_plan(ctypes.byref(pr), ctypes.byref(out)) == OK
    assert (out.segments, out.chunks_per_segment, out.walk_sums_prefix) == (4, 4, 1)
    # p = 32 packed state: the 528 unique (i, j) rows and 16 zero rows (34 tiles of 16) x 64,
    # + Z as four 16 x 16 tiles
    assert out.state_floats == 34 * 16 * 64 + 4 * 256
    for seg, n_seg, walk_sums in ((4, 8, 1), (3, 11, 0)):   # 32 chunks per sequence
        pr = _problem(B=1, H=2, T=2048)
        pr.seg_chunks = seg
        assert lib.kata_fwd_chunked_plan(ctypes.byref(pr), ctypes.byref(out)) == OK
        assert (out.segments, out.walk_sums_prefix) == (n_seg, walk_sums)
        assert (out.scan_levels == 0) == bool(walk_sums)
    # fp32 kernels: one state per chunk, a scan of ceil(log2 N_c) levels
    pr = _problem(B=1, H=1, T=256, p=8, dv=16, chunk=32, in_dt=0)
    assert lib.kata_fwd_chunked_plan(ctypes.byref(pr), ctypes.byref(out)) == OK
    assert (out.mfma, out.n_chunks, out.segments, out.scan_levels) == (0, 8, 8, 3)
    # errors
    assert lib.kata_fwd_chunked_plan(ctypes.byref(pr), None) == INVALID
    assert lib.kata_fwd_chunked_plan(ctypes.byref(_problem(T=100)), ctypes.byref(out)) == \
        UNSUPPORTED


def test_library_exports_only_the_declared_c_functions():
    # helpers stay internal: every exported C (unmangled) function is one of the header's
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", K.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.split()[1:2] == ["T"]}
    c_names = {n for n in exported if not n.startswith("_Z")}
    assert c_names <= set(_declared_functions()), sorted(c_names - set(_declared_functions()))


def test_noalloc_forward_rejects_a_problem_beyond_its_static_scratch():
    # validation runs before any device call: one state per chunk over 2 x 1024 chunks needs
    # more than the 64 MiB static scratch; the same problem with the default plan fits
    lib = _lib()
    q, k, v, o = _fake(4)
    big = _problem(B=1, H=2, T=65536, seg=1)
    assert lib.kata_fwd_chunked_workspace_size(ctypes.byref(big)) > K.NOALLOC_SCRATCH_BYTES
    assert lib.kata_fwd_chunked_noalloc(ctypes.byref(big), q, k, v, o, None, None) == WORKSPACE
    assert "static scratch" in lib.kata_last_error().decode()
    fits = _problem(B=1, H=2, T=65536)
    assert 0 < lib.kata_fwd_chunked_workspace_size(ctypes.byref(fits)) <= K.NOALLOC_SCRATCH_BYTES
    # argument errors as kata_fwd_chunked
    assert lib.kata_fwd_chunked_noalloc(None, q, k, v, o, None, None) == INVALID
    assert lib.kata_fwd_chunked_noalloc(ctypes.byref(_problem(T=100)), q, k, v, o, None,
                                        None) == UNSUPPORTED
    assert lib.kata_fwd_chunked_noalloc(ctypes.byref(fits), None, k, v, o, None, None) == INVALID


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define KATA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == K.NOALLOC_SCRATCH_BYTES


def test_strides_addressing_beyond_two_to_the_62_bytes_are_rejected():
    # every offset the kernels form must be exact in 64-bit arithmetic
    lib = _lib()
    pr = _problem(B=2, H=2, T=128)
    pr.sv[0] = 1 << 61                                   # (B - 1) * 2^61 elements of 2 bytes
    assert _chunked(pr) == INVALID and "2^62" in lib.kata_last_error().decode()
    pr = _problem(B=1, H=2, T=128)
    pr.sk[1] = (1 << 62) // 200                          # 127 * that * 2 bytes > 2^62 / 4 ...
    assert _quad(pr) == INVALID


def test_scan_rejects_a_states_array_beyond_two_to_the_62_bytes():
    lib = _lib()
    st = ctypes.c_void_p(FAKE)
    # 65535 sequences x 2^26 chunks x 2^30 floats: each size within its own cap
    assert lib.kata_chunk_state_scan(st, 65535, 1 << 26, 1 << 30, 1, None, None, 0, None,
                                     None) == INVALID
    assert "2^62" in lib.kata_last_error().decode()
    assert lib.kata_chunk_state_scan_workspace_size(65535, 1 << 26, 1 << 30) == 0
    assert lib.kata_chunk_state_scan_workspace_size(16, 48, 10496) == 0      # one tile
    assert lib.kata_chunk_state_scan_workspace_size(16, 5000, 10496) > 0     # tile totals


def test_parallel_kata_attn_has_no_cpu_path():
    # the differentiable op marshals into the same entry points: host tensors are refused
    # before anything reaches the library (there is no CPU fallback)
    import torch
    q = torch.randn(1, 64, 2, 16, dtype=torch.bfloat16)
    v = torch.randn(1, 64, 2, 64, dtype=torch.bfloat16)
    for form in ("auto", "chunked", "quadratic"):
        with pytest.raises(ValueError, match="GPU tensor"):
            K.parallel_kata_attn(q, q, v, form=form)


def test_parallel_kata_attn_dispatch_and_gradient_plumbing(monkeypatch):
    # the op's host logic with the library calls replaced by recorders (no arithmetic here):
    # "auto" takes the chunked forward where T is a multiple of the chunk, else the quadratic
    # one; the backward is the chunked one in the first case and the flash one in the second;
    # the output is requested in the inputs' dtype and the fp32 gradients come back in it
    import torch
    calls = []

    def fake_fwd(name):
        def f(q, k, v, **kw):
            calls.append((name, kw))
            return torch.full(v.shape, 0.5, dtype=kw["out_dtype"])
        return f

    def fake_bwd(q, k, v, dO, eps, chunk, groups):
        calls.append(("bwd", dict(chunk=chunk, groups=groups, eps=eps, dO_dtype=dO.dtype)))
        return (torch.full(q.shape, 1.0), torch.full(k.shape, 2.0), torch.full(v.shape, 3.0))

    monkeypatch.setattr(K, "fwd_chunked", fake_fwd("chunked"))
    monkeypatch.setattr(K, "fwd_quadratic", fake_fwd("quadratic"))
    monkeypatch.setattr(K, "bwd", fake_bwd)
    for T, fwd_name, bwd_chunk in ((128, "chunked", 64), (100, "quadratic", None)):
        calls.clear()
        q = torch.zeros(1, T, 2, 16, dtype=torch.bfloat16, requires_grad=True)
        k = torch.zeros(1, T, 2, 16, dtype=torch.bfloat16, requires_grad=True)
        v = torch.zeros(1, T, 2, 64, dtype=torch.bfloat16, requires_grad=True)
        o = K.parallel_kata_attn(q, k, v, num_groups=2, eps=1e-5)
        assert o.dtype == torch.bfloat16 and calls[0][0] == fwd_name
        assert calls[0][1]["groups"] == 2 and calls[0][1]["eps"] == 1e-5
        o.float().sum().backward()
        assert calls[1] == ("bwd", dict(chunk=bwd_chunk, groups=2, eps=1e-5,
                                         dO_dtype=torch.bfloat16))
        for x, val in ((q, 1.0), (k, 2.0), (v, 3.0)):
            assert x.grad.dtype == torch.bfloat16 and bool((x.grad == val).all())
    calls.clear()
    q = torch.zeros(1, 128, 2, 16, requires_grad=True)
    K.parallel_kata_attn(q, q, torch.zeros(1, 128, 2, 64), form="quadratic", chunk=32)
    assert calls[0][0] == "quadratic" and calls[0][1]["out_dtype"] == torch.float32

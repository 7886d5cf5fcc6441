"""Python binding of libkata: causal normalized linear attention with the rank-one PSD
feature map psi(u) = u u^T, hand-written HIP kernels for MI355X (gfx950).

Each function marshals torch tensors into the C ABI of include/kata.h and enqueues the work
on the current torch stream of the tensors' device; every step of the computation runs in
the library's kernels.  torch provides device memory and streams only.  There is no CPU
path: if libkata.so is missing, or a call fails, an exception is raised.

    o = fwd_chunked(q, k, v, chunk=64)          # exact O(T) chunked-state form
    o = fwd_quadratic(q, k, v)                  # flash-style O(T^2) form
    dq, dk, dv = bwd(q, k, v, dO)               # fp32 gradients of sum(dO * o)
    o = parallel_kata_attn(q, k, v)             # differentiable: forward + bwd under autograd
    levels, totals = chunk_state_scan(states)   # in-place exclusive prefix scan
    state = recurrent_state(k, v)               # (S, Z) after the given tokens (prefill)
    o = decode(q, k, v, state)                  # advance the state token by token

q, k: (B, T, H, p); v: (B, T, H, dv) -- the layout of the pages' kernel call -- with the last
dimension contiguous; any (b, t, h) strides that keep rows 16-byte aligned are accepted
(e.g. a head-major (B, H, T, D) tensor passed as .transpose(1, 2)).
"""

import ctypes
import os

import torch

__all__ = [
    "KataError", "parallel_kata_attn", "fwd_quadratic", "fwd_chunked", "fwd_chunked_noalloc", "chunked_workspace_size",
    "chunked_plan", "NOALLOC_SCRATCH_BYTES",
    "chunk_state_scan", "scan_workspace_size", "bwd", "bwd_workspace_size",
    "recurrent_state", "recurrent_state_workspace_size", "decode", "state_shape",
    "timing_begin", "timing_end", "library_path", "KERNEL_KINDS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkata.so")
_LIB = None

KATA_F32, KATA_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20     # KATA_NOALLOC_SCRATCH_BYTES of include/kata.h
KERNEL_KINDS = ("quadratic", "chunk_state", "scan", "chunk_output", "bwd", "decode",
                "state_sum")


class KataError(RuntimeError):
    def __init__(self, status, what, detail):
        self.status = status
        super().__init__(f"{what}: {detail}")


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("p", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("seg_chunks", ctypes.c_int32), ("state_layout", ctypes.c_int32),
        ("groups", ctypes.c_int32), ("eps", ctypes.c_float),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("sq", ctypes.c_int64 * 3), ("sk", ctypes.c_int64 * 3), ("sv", ctypes.c_int64 * 3),
        ("so", ctypes.c_int64 * 3), ("sdo", ctypes.c_int64 * 3),
    ]


class _ChunkedPlan(ctypes.Structure):
    _fields_ = [("n_chunks", ctypes.c_int64), ("chunks_per_segment", ctypes.c_int64),
                ("segments", ctypes.c_int64), ("state_floats", ctypes.c_int64),
                ("scan_levels", ctypes.c_int32), ("mfma", ctypes.c_int32),
                ("packed", ctypes.c_int32), ("walk_sums_prefix", ctypes.c_int32)]


class _Times(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * 7), ("total_ms", ctypes.c_double * 7)]


def library_path():
    return _LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; run `python -m kernelized_psd_feature_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, VP, SZ = ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_size_t
        I32, I64 = ctypes.c_int32, ctypes.c_int64
        sig = {
            "kata_fwd_quadratic": (I32, [P, VP, VP, VP, VP, VP, VP]),
            "kata_fwd_chunked_workspace_size": (SZ, [P]),
            "kata_fwd_chunked": (I32, [P, VP, VP, VP, VP, VP, VP, SZ, VP]),
            "kata_fwd_chunked_noalloc": (I32, [P, VP, VP, VP, VP, VP, VP]),
            "kata_fwd_chunked_plan": (I32, [P, ctypes.POINTER(_ChunkedPlan)]),
            "kata_chunk_state_scan_workspace_size": (SZ, [I64, I64, I64]),
            "kata_chunk_state_scan": (I32, [VP, I64, I64, I64, I32, VP, VP, SZ,
                                            ctypes.POINTER(I32), VP]),
            "kata_recurrent_state_workspace_size": (SZ, [P]),
            "kata_recurrent_state": (I32, [P, VP, VP, VP, VP, SZ, VP]),
            "kata_decode": (I32, [P, VP, VP, VP, VP, VP, VP, VP]),
            "kata_bwd_workspace_size": (SZ, [P]),
            "kata_bwd_chunked_workspace_size": (SZ, [P]),
            "kata_bwd_chunked": (I32, [P, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]),
            "kata_bwd": (I32, [P, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]),
            "kata_status_string": (ctypes.c_char_p, [I32]),
            "kata_last_error": (ctypes.c_char_p, []),
            "kata_timing_begin": (I32, []),
            "kata_timing_end": (I32, [ctypes.POINTER(_Times)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _LIB = lib
    return _LIB


def _check(status, what):
    if status != 0:
        lib = _lib()
        detail = (lib.kata_last_error() or b"").decode() or lib.kata_status_string(status).decode()
        raise KataError(status, what, f"{lib.kata_status_string(status).decode()} ({detail})")


def _dtype_code(dt):
    if dt == torch.float32:
        return KATA_F32
    if dt == torch.bfloat16:
        return KATA_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _bth_strides(x, name):
    if x.dim() != 4:
        raise ValueError(f"{name} must be 4-D (B, T, H, D)")
    if x.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")
    return (x.stride(0), x.stride(1), x.stride(2))


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


STATE_LAYOUTS = {"direct": 0, "packed": 1}


def _make_problem(q, k, v, o=None, dO=None, chunk=0, seg_chunks=0, eps=1e-6,
                  out_dtype=torch.float32, state="direct", groups=1):
    for name, x in (("q", q), ("k", k), ("v", v)):
        if not x.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    B, T, H, p = q.shape
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share (B, T, H) and dtype; q and k share p")
    pr = _Problem()
    pr.B, pr.H, pr.T, pr.p, pr.dv = B, H, T, p, v.shape[3]
    pr.chunk, pr.seg_chunks, pr.eps = chunk, seg_chunks, eps
    if state not in STATE_LAYOUTS:
        raise ValueError(f"state must be one of {sorted(STATE_LAYOUTS)}")
    pr.state_layout = STATE_LAYOUTS[state]
    pr.groups = groups
    pr.in_dtype, pr.out_dtype = _dtype_code(q.dtype), _dtype_code(out_dtype)
    pr.sq[:] = _bth_strides(q, "q")
    pr.sk[:] = _bth_strides(k, "k")
    pr.sv[:] = _bth_strides(v, "v")
    pr.so[:] = _bth_strides(o, "o") if o is not None else pr.sv[:]
    pr.sdo[:] = _bth_strides(dO, "dO") if dO is not None else pr.sv[:]
    return pr


def _out(q, v, out_dtype, out):
    if out is None:
        return torch.empty(v.shape, dtype=out_dtype, device=v.device)
    if out.shape != v.shape or out.dtype != out_dtype or out.device != v.device:
        raise ValueError("out must match v's shape and device and have out_dtype")
    return out


def fwd_quadratic(q, k, v, eps=1e-6, out_dtype=torch.float32, out=None, return_den=False,
                  groups=1):
    """Flash-style O(T^2) forward.  Returns o (and D_t = eps + sum_s a_ts, fp32 (B,T,H)).
    groups=g: KATA-Mg, a_ts = sum_j (q_t^(j) . k_s^(j))^2 over g consecutive coordinate
    groups (every public call takes this argument)."""
    o = _out(q, v, out_dtype, out)
    den = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_den else None
    pr = _make_problem(q, k, v, o, eps=eps, out_dtype=out_dtype, groups=groups)
    with torch.cuda.device(q.device):
        _check(_lib().kata_fwd_quadratic(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                         _ptr(den), _stream(q.device)), "kata_fwd_quadratic")
    return (o, den) if return_den else o


def chunked_workspace_size(q, k, v, chunk=64, seg_chunks=0, out_dtype=torch.float32,
                           state="packed", groups=1):
    pr = _make_problem(q, k, v, chunk=chunk, seg_chunks=seg_chunks, out_dtype=out_dtype,
                       state=state, groups=groups)
    return int(_lib().kata_fwd_chunked_workspace_size(ctypes.byref(pr)))


def chunked_plan(q, k, v, chunk=64, seg_chunks=0, out_dtype=torch.float32, state="packed",
                 groups=1):
    """The plan fwd_chunked takes (host only): n_chunks, chunks_per_segment, segments (per
    (b, h)), state_floats, scan_levels (0: no state pass and no scan), mfma, packed."""
    pr = _make_problem(q, k, v, chunk=chunk, seg_chunks=seg_chunks, out_dtype=out_dtype,
                       state=state, groups=groups)
    out = _ChunkedPlan()
    _check(_lib().kata_fwd_chunked_plan(ctypes.byref(pr), ctypes.byref(out)),
           "kata_fwd_chunked_plan")
    return {name: int(getattr(out, name)) for name, _ in _ChunkedPlan._fields_}


def fwd_chunked(q, k, v, chunk=64, eps=1e-6, out_dtype=torch.float32, seg_chunks=0,
                out=None, workspace=None, return_den=False, state="packed", groups=1):
    """Exact O(T) chunked-state forward (chunk states, prefix scan, readout).

    state: "packed" (the p(p+1)/2 unique state rows, the faster layout) or "direct" (all p^2
    rows); both give the same outputs up to rounding.
    workspace: optional preallocated uint8 GPU tensor of at least chunked_workspace_size()
    bytes (allocated here otherwise).  Returns o (and D_t if return_den)."""
    o = _out(q, v, out_dtype, out)
    den = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_den else None
    pr = _make_problem(q, k, v, o, chunk=chunk, seg_chunks=seg_chunks, eps=eps,
                       out_dtype=out_dtype, state=state, groups=groups)
    lib = _lib()
    need = int(lib.kata_fwd_chunked_workspace_size(ctypes.byref(pr)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        _check(lib.kata_fwd_chunked(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                    _ptr(den), _ptr(workspace), workspace.numel(),
                                    _stream(q.device)), "kata_fwd_chunked")
    return (o, den) if return_den else o


def fwd_chunked_noalloc(q, k, v, out, chunk=64, eps=1e-6, seg_chunks=0, den=None,
                        state="packed", groups=1):
    """fwd_chunked without a workspace: the library's static per-device scratch holds the
    segment states (problems whose workspace would exceed NOALLOC_SCRATCH_BYTES are rejected,
    except a spread p = 32 state pass that fits with one state per segment, which then runs
    that way and matches fwd_chunked to rounding).
    The caller passes the output `out` (its dtype is the output dtype) and optionally `den`
    (fp32 (B, T, H)); nothing is allocated.  Calls that overlap on one device race."""
    if out.shape != v.shape or out.device != v.device:
        raise ValueError("out must match v's shape and device")
    if den is not None and (den.shape != q.shape[:3] or den.dtype != torch.float32):
        raise ValueError("den must be fp32 (B, T, H)")
    pr = _make_problem(q, k, v, out, chunk=chunk, seg_chunks=seg_chunks, eps=eps,
                       out_dtype=out.dtype, state=state, groups=groups)
    with torch.cuda.device(q.device):
        _check(_lib().kata_fwd_chunked_noalloc(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(out), _ptr(den), _stream(q.device)),
               "kata_fwd_chunked_noalloc")
    return out


def scan_workspace_size(n_seq, n_chunks, state_elems):
    return int(_lib().kata_chunk_state_scan_workspace_size(n_seq, n_chunks, state_elems))


def chunk_state_scan(states, exclusive=True, want_totals=False, workspace=None):
    """In-place prefix scan of fp32 states shaped (n_seq, n_chunks, state_elems).

    Returns (levels, totals): the depth of the combining tree, and the inclusive totals
    (n_seq, state_elems) if want_totals else None."""
    if states.dtype != torch.float32 or states.dim() != 3 or not states.is_contiguous():
        raise ValueError("states must be a contiguous fp32 (n_seq, n_chunks, elems) tensor")
    n_seq, n, e = states.shape
    totals = torch.empty((n_seq, e), dtype=torch.float32, device=states.device) if want_totals else None
    lib = _lib()
    need = int(lib.kata_chunk_state_scan_workspace_size(n_seq, n, e))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=states.device)
    levels = ctypes.c_int32(-1)
    with torch.cuda.device(states.device):
        _check(lib.kata_chunk_state_scan(_ptr(states), n_seq, n, e, 1 if exclusive else 0,
                                         _ptr(totals), _ptr(workspace),
                                         0 if workspace is None else workspace.numel(),
                                         ctypes.byref(levels), _stream(states.device)),
               "kata_chunk_state_scan")
    return levels.value, totals


def state_shape(k, v):
    """Shape of the recurrent state of (B, T, H, p) keys and (B, T, H, dv) values:
    (B, H, dv + 1, p * p) fp32; [b, h, d] holds S[(i, j), d] at column i * p + j for d < dv
    and Z[i, j] for d = dv."""
    B, _, H, p = k.shape
    return (B, H, v.shape[-1] + 1, p * p)


def recurrent_state_workspace_size(k, v, chunk=64, groups=1):
    pr = _make_problem(k, k, v, chunk=chunk, groups=groups)
    return int(_lib().kata_recurrent_state_workspace_size(ctypes.byref(pr)))


def recurrent_state(k, v, chunk=64, out=None, workspace=None, groups=1):
    """Prefill: the state (S, Z) after all T tokens of k, v (T % chunk == 0), in the layout
    of state_shape()."""
    state = out if out is not None else torch.empty(state_shape(k, v), dtype=torch.float32,
                                                    device=k.device)
    if state.shape != state_shape(k, v) or state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 tensor of state_shape(k, v)")
    pr = _make_problem(k, k, v, chunk=chunk, groups=groups)
    lib = _lib()
    need = int(lib.kata_recurrent_state_workspace_size(ctypes.byref(pr)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=k.device)
    with torch.cuda.device(k.device):
        _check(lib.kata_recurrent_state(ctypes.byref(pr), _ptr(k), _ptr(v), _ptr(state),
                                        _ptr(workspace), workspace.numel(), _stream(k.device)),
               "kata_recurrent_state")
    return state


def decode(q, k, v, state, eps=1e-6, out_dtype=torch.float32, out=None, return_den=False,
           groups=1):
    """Advance `state` (in place) over the T tokens of q, k, v one at a time; returns o (and
    D_t).  T = 1 is one decode step."""
    if state.shape != state_shape(k, v) or state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 tensor of state_shape(k, v)")
    o = _out(q, v, out_dtype, out)
    den = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_den else None
    pr = _make_problem(q, k, v, o, eps=eps, out_dtype=out_dtype, groups=groups)
    with torch.cuda.device(q.device):
        _check(_lib().kata_decode(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(den), _ptr(state), _stream(q.device)), "kata_decode")
    return (o, den) if return_den else o


def bwd_workspace_size(q, k, v, groups=1):
    pr = _make_problem(q, k, v, groups=groups)
    return int(_lib().kata_bwd_workspace_size(ctypes.byref(pr)))


def bwd(q, k, v, dO, eps=1e-6, workspace=None, chunk=None, groups=1):
    """fp32 gradients (dq, dk, dv) of sum(dO * o), o the forward output.

    chunk=None: the flash-style O(T^2) backward; chunk=C: the chunked O(T) backward (forward
    prefix states for dq, a reverse scan of query states for dk and dv; T % C == 0)."""
    if dO.shape != v.shape or dO.dtype != q.dtype:
        raise ValueError("dO must match v's shape and q's dtype")
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    # gradient outputs share the strides of their inputs
    qs, ks, vs = (q, k, v) if q.is_contiguous() and k.is_contiguous() and v.is_contiguous() \
        else (q.contiguous(), k.contiguous(), v.contiguous())
    pr = _make_problem(qs, ks, vs, dO=dO, eps=eps, chunk=chunk or 0, groups=groups)
    lib = _lib()
    size_fn, fn, name = ((lib.kata_bwd_workspace_size, lib.kata_bwd, "kata_bwd") if chunk is None
                         else (lib.kata_bwd_chunked_workspace_size, lib.kata_bwd_chunked,
                               "kata_bwd_chunked"))
    need = int(size_fn(ctypes.byref(pr)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        _check(fn(ctypes.byref(pr), _ptr(qs), _ptr(ks), _ptr(vs), _ptr(dO), _ptr(dq), _ptr(dk),
                  _ptr(dv), _ptr(workspace), workspace.numel(), _stream(q.device)), name)
    return dq, dk, dv


class _KataAttn(torch.autograd.Function):
    """fwd_chunked / fwd_quadratic as the forward and bwd as the backward of one autograd node.
    Only the inputs are kept for the backward, which recomputes what it needs in the library."""

    @staticmethod
    def forward(ctx, q, k, v, num_groups, form, chunk, eps):
        if form == "chunked":
            o = fwd_chunked(q, k, v, chunk=chunk, eps=eps, out_dtype=q.dtype, groups=num_groups)
        else:
            o = fwd_quadratic(q, k, v, eps=eps, out_dtype=q.dtype, groups=num_groups)
        ctx.save_for_backward(q, k, v)
        # the chunked O(T) backward where T is a multiple of the chunk, else the flash one
        ctx.cfg = (num_groups, chunk if q.shape[1] % chunk == 0 else None, eps)
        return o

    @staticmethod
    def backward(ctx, dO):
        q, k, v = ctx.saved_tensors
        groups, chunk, eps = ctx.cfg
        dq, dk, dv = bwd(q, k, v, dO.contiguous(), eps=eps, chunk=chunk, groups=groups)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None, None


def parallel_kata_attn(q, k, v, num_groups=1, form="auto", chunk=64, eps=1e-6):
    """Causal KATA attention as a differentiable op: (B, T, H, D) -> (B, T, H, d_v), the
    output in the inputs' dtype, named and laid out like the KATA README's kernel call
    (num_groups: the KATA-Mg factor count g).

    form: "chunked" (exact O(T) chunked-state forward; T a multiple of chunk), "quadratic"
    (flash-style O(T^2)), or "auto" (chunked where T is a multiple of chunk, else quadratic).
    Under autograd the backward runs bwd (chunked where T is a multiple of chunk, else flash);
    its fp32 gradients are handed back in the inputs' dtype."""
    if form == "auto":
        form = "chunked" if q.shape[1] % chunk == 0 else "quadratic"
    if form not in ("chunked", "quadratic"):
        raise ValueError("form must be 'auto', 'chunked' or 'quadratic'")
    return _KataAttn.apply(q, k, v, num_groups, form, chunk, eps)


def timing_begin():
    _check(_lib().kata_timing_begin(), "kata_timing_begin")


def timing_end():
    """Returns {kind: (launches, total_ms)} for the kernels enqueued since timing_begin()."""
    t = _Times()
    _check(_lib().kata_timing_end(ctypes.byref(t)), "kata_timing_end")
    return {name: (int(t.launches[i]), float(t.total_ms[i])) for i, name in enumerate(KERNEL_KINDS)}

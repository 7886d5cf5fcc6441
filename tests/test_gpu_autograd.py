"""parallel_kata_attn, the differentiable op over the C ABI: its forward is the library's
forward with the output in the inputs' dtype, its gradients under torch autograd are the
library's backward (bit for bit, once handed back in the inputs' dtype), and both agree with
the fp64 oracle (max-abs 1e-2 for bf16 inputs, 1e-4 for fp32 inputs, beyond the rounding of
a bf16 result to bf16)."""

import sys

import numpy as np
import pytest
import torch

import kata_workloads as W
import kernelized_psd_feature_amd as K
import oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _np(x):
    return x.detach().to(torch.float64).cpu().numpy()


def _leaf(x):
    return x.to(DEV).requires_grad_(True)


def _err(got, ref):
    """max |got - ref| beyond a bf16 result's own rounding for bf16 tensors (round to nearest
    with 8 significant bits: at most half an ulp, 2^-8 of the value's magnitude, for values
    just above a power of two); plain max-abs for fp32 ones"""
    g = got.detach().to(torch.float64).cpu().numpy()
    slack = 2.0 ** -8 * np.abs(ref) if got.dtype == torch.bfloat16 else 0.0
    return float(np.max(np.abs(g - ref) - slack))


@pytest.mark.parametrize("form,groups,T", [("auto", 1, 256), ("quadratic", 1, 256),
                                           ("auto", 2, 256), ("auto", 1, 200)])
def test_parallel_kata_attn_bf16_forward_and_autograd(form, groups, T):
    # the training recipe (bf16, p = 16, d_v = 64); T = 200 is not a multiple of the chunk, so
    # "auto" takes the quadratic forward and the flash backward there
    w = W.WORKLOADS[5]
    q, k, v, g = W.make_inputs(w, 41, T=T, B=2, H=4, with_dO=True)
    ql, kl, vl = _leaf(q), _leaf(k), _leaf(v)
    o = K.parallel_kata_attn(ql, kl, vl, num_groups=groups, form=form)
    assert o.dtype == torch.bfloat16 and o.shape == v.shape
    o.backward(g.to(DEV))
    torch.cuda.synchronize()

    chunked = form == "auto" and T % 64 == 0
    qd, kd, vd, gd = (x.to(DEV) for x in (q, k, v, g))
    want = (K.fwd_chunked(qd, kd, vd, chunk=64, out_dtype=torch.bfloat16, groups=groups)
            if chunked else K.fwd_quadratic(qd, kd, vd, out_dtype=torch.bfloat16, groups=groups))
    assert torch.equal(o.detach(), want)
    grads = K.bwd(qd, kd, vd, gd, chunk=64 if T % 64 == 0 else None, groups=groups)
    for leaf, gr in zip((ql, kl, vl), grads):
        assert leaf.grad.dtype == torch.bfloat16
        assert torch.equal(leaf.grad, gr.to(torch.bfloat16))

    ref_o, _ = O.closed_form(_np(q), _np(k), _np(v), groups=groups)
    refs = O.backward(_np(q), _np(k), _np(v), _np(g), groups=groups)
    e_o = _err(o, ref_o)
    e_g = [_err(leaf.grad, r) for leaf, r in zip((ql, kl, vl), refs)]
    say(f"parallel_kata_attn {form} g={groups} T={T}: o {e_o:.3e}, dq/dk/dv {e_g}")
    assert e_o <= 1e-2 and max(e_g) <= 1e-2


@pytest.mark.parametrize("form", ["auto", "quadratic"])
def test_parallel_kata_attn_fp32_autograd(form):
    # the tiny fp32 recipe (p = 8, d_v = 16), chunk 32
    w = W.WORKLOADS[1]
    q, k, v, g = W.make_inputs(w, 42, B=1, H=2, with_dO=True)
    ql, kl, vl = _leaf(q), _leaf(k), _leaf(v)
    o = K.parallel_kata_attn(ql, kl, vl, form=form, chunk=32)
    assert o.dtype == torch.float32
    (o * g.to(DEV)).sum().backward()
    torch.cuda.synchronize()
    ref_o, _ = O.closed_form(_np(q), _np(k), _np(v))
    refs = O.backward(_np(q), _np(k), _np(v), _np(g))
    scale = max(1.0, max(float(np.abs(r).max()) for r in refs))
    e_g = [_err(leaf.grad, r) for leaf, r in zip((ql, kl, vl), refs)]
    say(f"parallel_kata_attn fp32 {form}: o {_err(o, ref_o):.3e}, dq/dk/dv {e_g} "
        f"(scale {scale:.2f})")
    assert _err(o, ref_o) <= 1e-4 and max(e_g) <= 1e-4 * scale


def test_parallel_kata_attn_grads_only_where_asked():
    # q and k constants, v a leaf: only v receives a gradient, the library's dv
    w = W.WORKLOADS[5]
    q, k, v, g = (x.to(DEV) for x in W.make_inputs(w, 43, T=128, B=1, H=2, with_dO=True))
    vl = v.clone().requires_grad_(True)
    K.parallel_kata_attn(q, k, vl).backward(g)
    torch.cuda.synchronize()
    assert q.grad is None and k.grad is None
    assert torch.equal(vl.grad, K.bwd(q, k, v, g, chunk=64)[2].to(torch.bfloat16))


def test_parallel_kata_attn_rejects_an_unknown_form():
    w = W.WORKLOADS[5]
    q, k, v = (x.to(DEV) for x in W.make_inputs(w, 44, T=64, B=1, H=1))
    with pytest.raises(ValueError):
        K.parallel_kata_attn(q, k, v, form="linear")

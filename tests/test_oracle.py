"""Pins for the CPU oracle: each oracle function is checked against something other than
itself -- values the pages print, a hand-worked example, textbook special cases with closed
forms, library routines, invariants of the method, and finite differences.

Runs on the CPU only (no GPU marker)."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(rng, B, T, H, p, dv, unit_k=True, unit_q=True):
    q = rng.standard_normal((B, T, H, p))
    k = rng.standard_normal((B, T, H, p))
    v = rng.standard_normal((B, T, H, dv))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    if unit_q:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    return q, k, v


def _forms():
    """Every oracle route to the forward output, as f(q, k, v, eps) -> (o, D)."""
    def rows(q, k, v, eps):
        B, T, H, _ = q.shape
        o = np.empty((B, T, H, v.shape[-1]))
        d = np.empty((B, T, H))
        for b in range(B):
            for h in range(H):
                r = np.arange(T)[::-1].copy()           # any order of rows
                ob, db = O.closed_form_rows(q[b, :, h], k[b, :, h], v[b, :, h], r, eps, block=3)
                o[b, r, h] = ob
                d[b, r, h] = db
        return o, d

    def chunk_any(C):
        def f(q, k, v, eps):
            T = q.shape[1]
            c = C if T % C == 0 else 1
            return O.chunked(q, k, v, c, eps)
        return f

    return {
        "closed_form": lambda q, k, v, eps: O.closed_form(q, k, v, eps),
        "closed_form_block3": lambda q, k, v, eps: O.closed_form(q, k, v, eps, block=3),
        "closed_form_rows": rows,
        "recurrent": O.recurrent,
        "chunked_C1": chunk_any(1),
        "chunked_C2": chunk_any(2),
        "chunked_C4": chunk_any(4),
    }


FORMS = _forms()


# ---------------------------------------------------------------- feature map ----------

@pytest.mark.parametrize("p", [1, 2, 3, 4, 8, 16, 32])
def test_feature_inner_product_squares_raw_inner_product_exactly(p):
    # gist.science 2.2 / ai.info squaring bullet: <psi(q), psi(k)> = (q . k)^2.  With small
    # integers every product and sum is exact in float64, so equality is bitwise.
    rng = np.random.default_rng(p)
    for _ in range(50):
        q = rng.integers(-3, 4, size=p).astype(np.float64)
        k = rng.integers(-3, 4, size=p).astype(np.float64)
        assert O.feature(q) @ O.feature(k) == (q @ k) ** 2


def test_feature_layout_row_major():
    u = np.array([2.0, 3.0, 5.0])
    np.testing.assert_array_equal(O.feature(u), [4, 6, 10, 6, 9, 15, 10, 15, 25])


def test_feature_widths_match_printed_values():
    g = _load("state_sizes.json")
    u = np.random.default_rng(0).standard_normal(64)
    f = O.feature(u)
    assert f.size == g["direct_width_d64"]["value"]
    # a generic u gives exactly d(d+1)/2 distinct coordinates (the packed width)
    assert np.unique(f).size == g["packed_width_d64"]["value"]


def test_state_elems_matches_printed_state_size():
    g = _load("state_sizes.json")
    assert O.state_elems(64, 64) == g["m1_state_entries_d64_dv64"]["value"]


# ---------------------------------------------------------------- worked example -------

@pytest.mark.parametrize("form", list(FORMS))
def test_hand_worked_example(form):
    g = _load("hand_worked_example.json")
    eps = g["eps"]
    q = np.array(g["q"], float)[None, :, None, :]
    k = np.array(g["k"], float)[None, :, None, :]
    v = np.array(g["v"], float)[None, :, None, :]
    o, d = FORMS[form](q, k, v, eps)
    den = np.array(g["denominator_minus_eps"], float) + eps
    want = np.array(g["numerator"], float) / den[:, None]
    np.testing.assert_allclose(o[0, :, 0], want, rtol=1e-14, atol=0)
    np.testing.assert_allclose(d[0, :, 0], den, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- special cases --------

@pytest.mark.parametrize("form", list(FORMS))
def test_p1_is_weighted_prefix_mean(form):
    # p = 1: a[t,s] = q_t^2 k_s^2, so o_t = q_t^2 cumsum(k^2 v)_t / (eps + q_t^2 cumsum(k^2)_t)
    rng = np.random.default_rng(1)
    T, dv, eps = 16, 3, 1e-6
    q = rng.standard_normal((1, T, 1, 1))
    k = rng.standard_normal((1, T, 1, 1))
    v = rng.standard_normal((1, T, 1, dv))
    o, d = FORMS[form](q, k, v, eps)
    q2 = q[0, :, 0, 0] ** 2
    k2 = k[0, :, 0, 0] ** 2
    num = q2[:, None] * np.cumsum(k2[:, None] * v[0, :, 0], axis=0)
    den = eps + q2 * np.cumsum(k2)
    np.testing.assert_allclose(o[0, :, 0], num / den[:, None], rtol=1e-12)
    np.testing.assert_allclose(d[0, :, 0], den, rtol=1e-12)


@pytest.mark.parametrize("form", list(FORMS))
def test_identical_unit_keys_give_causal_running_mean(form):
    # all q_t = k_s = e_1: a = 1 for s <= t, so o_t = (sum_{s<=t} v_s) / (t + 1 + eps)
    rng = np.random.default_rng(2)
    T, p, dv, eps = 16, 4, 5, 1e-6
    q = np.zeros((1, T, 1, p)); q[..., 0] = 1
    k = q.copy()
    v = rng.standard_normal((1, T, 1, dv))
    o, _ = FORMS[form](q, k, v, eps)
    want = np.cumsum(v[0, :, 0], axis=0) / (np.arange(T) + 1 + eps)[:, None]
    np.testing.assert_allclose(o[0, :, 0], want, rtol=1e-13)


@pytest.mark.parametrize("form", list(FORMS))
def test_eps_is_added_once_outside_the_sum(form):
    # keys e_1, queries sqrt(eps) e_1: every a[t,s] = eps, so
    # o_t = eps sum v / (eps + (t+1) eps) = sum_{s<=t} v_s / (t + 2).
    rng = np.random.default_rng(3)
    T, p, dv, eps = 16, 3, 2, 1e-6
    k = np.zeros((1, T, 1, p)); k[..., 0] = 1
    q = k * np.sqrt(eps)
    v = rng.standard_normal((1, T, 1, dv))
    o, _ = FORMS[form](q, k, v, eps)
    want = np.cumsum(v[0, :, 0], axis=0) / (np.arange(T) + 2.0)[:, None]
    np.testing.assert_allclose(o[0, :, 0], want, rtol=1e-9)


@pytest.mark.parametrize("form", list(FORMS))
def test_orthonormal_keys_retrieve_exactly(form):
    # T <= p orthonormal keys (a permuted basis); q_t = k_{j(t)} with j(t) <= t.  Then only
    # s = j(t) scores (1), so o_t = v_{j(t)} / (1 + eps).
    rng = np.random.default_rng(4)
    T, p, dv, eps = 8, 8, 3, 1e-6
    basis = np.eye(p)[rng.permutation(p)]
    k = basis[:T][None, :, None, :]
    j = np.array([rng.integers(0, t + 1) for t in range(T)])
    q = k[:, j]
    v = rng.standard_normal((1, T, 1, dv))
    o, d = FORMS[form](q, k, v, eps)
    np.testing.assert_allclose(o[0, :, 0], v[0, j, 0] / (1 + eps), rtol=1e-14)
    np.testing.assert_allclose(d[0, :, 0], 1 + eps, rtol=1e-15)


@pytest.mark.parametrize("form", list(FORMS))
def test_zero_query_gives_zero(form):
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 1, 8, 2, 3, 2)
    q[:] = 0
    o, d = FORMS[form](q, k, v, 1e-6)
    assert np.all(o == 0)
    np.testing.assert_allclose(d, 1e-6, rtol=1e-15)


# ---------------------------------------------------------------- invariants -----------

@pytest.mark.parametrize("form", list(FORMS))
def test_weights_nonnegative_causal_and_sum_to_one_minus_eps_over_D(form):
    # With v = I (d_v = T) the output row o_t IS the weight row w[t, s] = a[t,s] / D_t.
    rng = np.random.default_rng(6)
    T, p, eps = 12, 3, 1e-6
    q, k, _ = _rand(rng, 1, T, 1, p, 1)
    v = np.eye(T)[None, :, None, :]
    w, d = FORMS[form](q, k, v, eps)
    w = w[0, :, 0]
    d = d[0, :, 0]
    assert np.all(w >= -1e-15)
    assert np.all(np.triu(w, 1) == 0)                     # no weight on future tokens
    np.testing.assert_allclose(w.sum(axis=1), 1 - eps / d, rtol=1e-13)


@pytest.mark.parametrize("form", list(FORMS))
def test_output_lies_in_hull_of_past_values_and_zero(form):
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 2, 16, 2, 4, 3)
    o, _ = FORMS[form](q, k, v, 1e-6)
    lo = np.minimum(0, np.minimum.accumulate(v, axis=1))
    hi = np.maximum(0, np.maximum.accumulate(v, axis=1))
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


@pytest.mark.parametrize("form", list(FORMS))
def test_future_tokens_never_reach_earlier_outputs(form):
    # Tokens after position t (even NaN/Inf ones) leave o_{<=t} bitwise unchanged.
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 1, 12, 1, 3, 2)
    o1, _ = FORMS[form](q, k, v, 1e-6)
    k2, v2 = k.copy(), v.copy()
    k2[:, 7:] = np.nan
    v2[:, 7:] = np.inf
    o2, _ = FORMS[form](q, k2, v2, 1e-6)
    np.testing.assert_array_equal(o1[:, :7], o2[:, :7])


@pytest.mark.parametrize("form", list(FORMS))
def test_permuting_the_past_leaves_the_output_unchanged(form):
    # The state update is additive and commutative (ai.info gate bullet): reordering tokens
    # s < t (keys with their values) does not change o_t.
    rng = np.random.default_rng(9)
    T = 12
    q, k, v = _rand(rng, 1, T, 1, 4, 3)
    perm = np.concatenate([rng.permutation(T - 1), [T - 1]])
    o1, _ = FORMS[form](q, k, v, 1e-6)
    o2, _ = FORMS[form](q, k[:, perm], v[:, perm], 1e-6)
    np.testing.assert_allclose(o1[:, T - 1], o2[:, T - 1], rtol=1e-12)


def test_gate_is_convex_and_reproduces_output():
    # ai.info gate bullet / gist.science 2.1: o_t = alpha_t ohat_{t-1} + beta_t v_t,
    # alpha_t + beta_t = 1, both in [0, 1].
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 2, 20, 2, 4, 3)
    o, _ = O.closed_form(q, k, v)
    a, b, oh = O.gate_terms(q, k, v)
    np.testing.assert_allclose(a + b, 1.0, rtol=0, atol=4.5e-16)   # 2 ulp
    assert np.all((a >= 0) & (a <= 1) & (b >= 0) & (b <= 1))
    np.testing.assert_allclose(a[..., None] * oh + b[..., None] * v, o, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- forms agree ----------

@settings(max_examples=25, deadline=None)
@given(T=st.integers(1, 24), p=st.integers(1, 5), dv=st.integers(1, 4),
       seed=st.integers(0, 2**31 - 1), unit=st.booleans())
def test_all_forms_agree(T, p, dv, seed, unit):
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, T, 2, p, dv, unit_k=unit, unit_q=unit)
    o_ref, d_ref = O.closed_form(q, k, v)
    o_rec, d_rec = O.recurrent(q, k, v)
    # q^T Z q sums products of both signs: its fp64 rounding error is bounded by a small
    # multiple of u * sum_s (|q_t| . |k_s|)^2 (u = 2^-53), which dominates rtol when D_t ~ eps
    qa, ka = np.abs(q[0].transpose(1, 0, 2)), np.abs(k[0].transpose(1, 0, 2))
    mag = np.cumsum(np.einsum("htp,hsp->hts", qa, ka) ** 2 * np.tril(np.ones((T, T))), axis=2)
    d_tol = 64 * 2.0 ** -53 * np.diagonal(mag, axis1=1, axis2=2).T[None]
    np.testing.assert_allclose(o_rec, o_ref, rtol=1e-10, atol=1e-12)
    assert np.all(np.abs(d_rec - d_ref) <= 1e-12 * np.abs(d_ref) + d_tol)
    for C in [c for c in range(1, T + 1) if T % c == 0]:
        o_ch, d_ch = O.chunked(q, k, v, C)
        np.testing.assert_allclose(o_ch, o_ref, rtol=1e-10, atol=1e-12)
        assert np.all(np.abs(d_ch - d_ref) <= 1e-12 * np.abs(d_ref) + d_tol)


def test_chunk_equal_to_T_is_the_quadratic_block():
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 2, 32, 3, 4, 5)
    o1, d1 = O.chunked(q, k, v, 32)
    o2, d2 = O.closed_form(q, k, v, block=32)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=0)
    np.testing.assert_allclose(d1, d2, rtol=1e-15)


def test_closed_form_rows_match_full():
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 1, 300, 1, 4, 3)
    o, d = O.closed_form(q, k, v)
    rows = rng.choice(300, 40, replace=False)
    orow, drow = O.closed_form_rows(q[0, :, 0], k[0, :, 0], v[0, :, 0], rows, block=7)
    np.testing.assert_allclose(orow, o[0, rows, 0], rtol=1e-13)
    np.testing.assert_allclose(drow, d[0, rows, 0], rtol=1e-14)


def test_chunked_rejects_ragged_T():
    q = np.zeros((1, 10, 1, 2))
    with pytest.raises(ValueError):
        O.chunked(q, q, q, 4)


# ---------------------------------------------------------------- chunk states, scan ---

def test_chunk_states_contract_to_squared_scores():
    # feature(q) . dS_c = sum_{s in c} (q . k_s)^2 v_s and q^T dZ_c q = sum_{s in c} (q . k_s)^2,
    # each computed here from raw inner products; dS is symmetric in its (i, j) feature pair.
    rng = np.random.default_rng(13)
    B, T, H, p, dv, C = 2, 24, 2, 4, 3, 8
    _, k, v = _rand(rng, B, T, H, p, dv)
    dS, dZ = O.chunk_states(k, v, C)
    x = rng.standard_normal(p)
    for b in range(B):
        for h in range(H):
            for c in range(T // C):
                K = k[b, c * C:(c + 1) * C, h]
                V = v[b, c * C:(c + 1) * C, h]
                s2 = (K @ x) ** 2
                np.testing.assert_allclose(O.feature(x) @ dS[b, h, c], s2 @ V, rtol=1e-12)
                np.testing.assert_allclose(x @ dZ[b, h, c] @ x, s2.sum(), rtol=1e-12)
                m = dS[b, h, c].reshape(p, p, dv)
                np.testing.assert_array_equal(m, m.transpose(1, 0, 2))
                np.testing.assert_allclose(np.trace(dZ[b, h, c]), (K * K).sum(), rtol=1e-13)


def test_exclusive_scan_matches_cumsum():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((2, 3, 17, 5))
    ex, tot = O.exclusive_scan(x, axis=2)
    cs = np.cumsum(x, axis=2)
    np.testing.assert_allclose(ex, cs - x, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(tot, cs[:, :, -1], rtol=1e-13)
    assert np.all(ex[:, :, 0] == 0)
    np.testing.assert_allclose(np.diff(ex, axis=2), x[:, :, :-1], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- backward -------------

def _loss(q, k, v, dO, eps):
    o, _ = O.closed_form(q, k, v, eps)
    return float((o * dO).sum())


@pytest.mark.parametrize("eps,unit", [(1e-2, False), (1e-6, True)])
def test_backward_matches_central_finite_differences(eps, unit):
    rng = np.random.default_rng(15)
    B, T, H, p, dv = 1, 10, 2, 3, 2
    q, k, v = _rand(rng, B, T, H, p, dv, unit_k=unit, unit_q=unit)
    if unit:                                   # keep every D_t >> eps
        q *= 2.0
    dO = rng.standard_normal((B, T, H, dv))
    dq, dk, dv_ = O.backward(q, k, v, dO, eps)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv_)):
        num = np.empty_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(**args_p, dO=dO, eps=eps) - _loss(**args_m, dO=dO, eps=eps)) / (2 * h)
        scale = max(1.0, np.abs(num).max())
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-6 * scale, err_msg=name)


def _autograd_closed_form_grads(q, k, v, dO, eps, groups):
    """Gradients of L = sum <dO, o> by torch float64 autograd of the closed form
    o_t = sum_{s<=t} a_ts v_s / (eps + sum_{s<=t} a_ts), a_ts = sum_j (q_t^(j) . k_s^(j))^2,
    written here in torch: a second route to the derivative, independent of the hand-derived
    formulas of oracle.backward."""
    import torch

    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    tdO = torch.tensor(dO, dtype=torch.float64)
    B, T, H, p = q.shape
    w = p // groups
    loss = 0.0
    for b in range(B):
        for h in range(H):
            Q, K, V = tq[b, :, h], tk[b, :, h], tv[b, :, h]
            a = 0.0
            for j in range(groups):
                sc = Q[:, j * w:(j + 1) * w] @ K[:, j * w:(j + 1) * w].T
                a = a + sc * sc
            a = torch.tril(a)
            o = (a @ V) / (eps + a.sum(dim=1, keepdim=True))
            loss = loss + (o * tdO[b, :, h]).sum()
    return [g.numpy() for g in torch.autograd.grad(loss, (tq, tk, tv))]


@pytest.mark.parametrize("groups", [1, 2, 4])
def test_backward_matches_float64_autograd_of_the_closed_form(groups):
    # the training workload's head shape (p = 16, d_v = 64) on a T = 256 slice, unit rows with
    # q scaled by 2 so every D_t >> eps (the gradients grow like 1 / D_t)
    rng = np.random.default_rng(31 + groups)
    q, k, v = _rand(rng, 2, 256, 2, 16, 64)
    q *= 2.0
    dO = rng.standard_normal(v.shape)
    eps = O.EPS
    hand = O.backward(q, k, v, dO, eps, groups=groups)
    auto = _autograd_closed_form_grads(q, k, v, dO, eps, groups)
    for name, x, y in zip(("dq", "dk", "dv"), hand, auto):
        scale = np.abs(y).max()
        np.testing.assert_allclose(x, y, rtol=1e-10, atol=1e-12 * scale, err_msg=name)


def test_backward_tiling_is_invisible():
    rng = np.random.default_rng(16)
    q, k, v = _rand(rng, 1, 40, 2, 4, 3)
    dO = rng.standard_normal(v.shape)
    a = O.backward(q, k, v, dO, block=512)
    b = O.backward(q, k, v, dO, block=7)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)


def test_backward_causality():
    # a perturbation of dO_t changes dv_s only for s <= t, and dq only at row t
    rng = np.random.default_rng(17)
    q, k, v = _rand(rng, 1, 12, 1, 3, 2)
    dO = rng.standard_normal(v.shape)
    dq1, dk1, dv1 = O.backward(q, k, v, dO)
    dO2 = dO.copy()
    dO2[:, 5] += 1.0
    dq2, dk2, dv2 = O.backward(q, k, v, dO2)
    np.testing.assert_array_equal(dv1[:, 6:], dv2[:, 6:])
    np.testing.assert_array_equal(dk1[:, 6:], dk2[:, 6:])
    np.testing.assert_array_equal(np.delete(dq1, 5, axis=1), np.delete(dq2, 5, axis=1))


# ------------------------------------------------------------ KATA-Mg (groups) ----------

def _orthant_closed_form(q, k, v, eps):
    """groups = p: every group is one coordinate, so a_ts = sum_i q_i^2 k_i^2 -- linear
    attention with the positive-orthant feature u*u, written out directly."""
    B, T, H, _ = q.shape
    o = np.empty((B, T, H, v.shape[-1]))
    d = np.empty((B, T, H))
    for b in range(B):
        for h in range(H):
            W = np.tril((q[b, :, h] ** 2) @ (k[b, :, h] ** 2).T)
            d[b, :, h] = eps + W.sum(axis=1)
            o[b, :, h] = (W @ v[b, :, h]) / d[b, :, h][:, None]
    return o, d


def _all_grouped_forms(q, k, v, eps, g):
    T = q.shape[1]
    out = {"closed_form": O.closed_form(q, k, v, eps, block=5, groups=g),
           "recurrent": O.recurrent(q, k, v, eps, groups=g),
           "chunked": O.chunked(q, k, v, 4 if T % 4 == 0 else T, eps, groups=g)}
    B, _, H, _ = q.shape
    o = np.empty((B, T, H, v.shape[-1]))
    d = np.empty((B, T, H))
    rows = np.arange(T)[::-1]
    for b in range(B):
        for h in range(H):
            ob, db = O.closed_form_rows(q[b, :, h], k[b, :, h], v[b, :, h], rows, eps,
                                        block=3, groups=g)
            o[b, rows, h], d[b, rows, h] = ob, db
    out["closed_form_rows"] = (o, d)
    return out


@pytest.mark.parametrize("p", [4, 8])
def test_groups_equal_p_is_the_positive_orthant_feature(p):
    rng = np.random.default_rng(40 + p)
    q, k, v = _rand(rng, 2, 12, 2, p, 3, unit_q=False)
    want = _orthant_closed_form(q, k, v, 1e-6)
    for name, (o, d) in _all_grouped_forms(q, k, v, 1e-6, p).items():
        np.testing.assert_allclose(o, want[0], rtol=1e-11, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(d, want[1], rtol=1e-11, err_msg=name)


@pytest.mark.parametrize("p,g", [(8, 2), (8, 4), (16, 2), (6, 3)])
def test_grouped_output_is_sum_of_per_group_numerators_over_shared_denominator(p, g):
    # a_ts = sum_j a_ts^(j), so N_t = sum_j N_t^(j) and D_t - eps = sum_j (D_t^(j) - eps),
    # each per-group term being the ungrouped closed form on that group's coordinates
    rng = np.random.default_rng(50 + p + g)
    q, k, v = _rand(rng, 1, 14, 2, p, 5)
    eps = 1e-3
    num = 0.0
    dsum = 0.0
    w = p // g
    for j in range(g):
        sl = slice(j * w, (j + 1) * w)
        oj, dj = O.closed_form(q[..., sl], k[..., sl], v, eps)
        num = num + oj * dj[..., None]
        dsum = dsum + (dj - eps)
    want_d = eps + dsum
    want_o = num / want_d[..., None]
    for name, (o, d) in _all_grouped_forms(q, k, v, eps, g).items():
        np.testing.assert_allclose(o, want_o, rtol=1e-10, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(d, want_d, rtol=1e-12, err_msg=name)


def test_grouped_feature_inner_product_is_sum_of_group_squares_exactly():
    rng = np.random.default_rng(60)
    for p, g in [(8, 2), (16, 4), (32, 2), (12, 3)]:
        q = rng.integers(-3, 4, size=(50, p)).astype(np.float64)
        k = rng.integers(-3, 4, size=(50, p)).astype(np.float64)
        got = (O.feature(q, g) * O.feature(k, g)).sum(axis=-1)
        w = p // g
        want = sum((q[:, j * w:(j + 1) * w] * k[:, j * w:(j + 1) * w]).sum(axis=-1) ** 2
                   for j in range(g))
        assert np.array_equal(got, want)
        assert O.feature(q, g).shape[-1] == p * p // g


def test_grouped_packed_widths_match_printed_state_sizes():
    g = _load("state_sizes.json")
    assert O.packed_width(64, 1) == g["packed_width_d64"]["value"]
    assert O.packed_width(64, 2) == g["mg_packed_width_formula"]["value_d64_g2"]
    # the review's entry counts: twice the packed state, d_v = 64
    assert 2 * O.packed_width(64, 1) * 64 == g["m1_state_entries_d64_dv64"]["value"]
    assert 2 * O.packed_width(64, 2) * 64 == g["m2_state_entries_d64_dv64"]["value"]
    for d in (8, 16, 32, 64):
        for gg in (1, 2, 4):
            assert O.packed_width(d, gg) == d * (d // gg + 1) // 2


def test_grouped_chunk_states_are_per_group_outer_products():
    rng = np.random.default_rng(61)
    p, g, C = 8, 2, 4
    _, k, v = _rand(rng, 1, 8, 1, p, 3)
    dS, dZ = O.chunk_states(k, v, C, groups=g)
    assert dS.shape == (1, 1, 2, p * p // g, 3)
    for c in range(2):
        Kc, Vc = k[0, c * C:(c + 1) * C, 0], v[0, c * C:(c + 1) * C, 0]
        rows = []
        for j in range(g):
            blk = Kc[:, j * 4:(j + 1) * 4]
            rows.append(np.einsum("si,sj,sd->ijd", blk, blk, Vc).reshape(16, 3))
        np.testing.assert_allclose(dS[0, 0, c], np.concatenate(rows), rtol=1e-13, atol=1e-15)
        Zfull = Kc.T @ Kc
        assert np.all(dZ[0, 0, c][:4, 4:] == 0) and np.all(dZ[0, 0, c][4:, :4] == 0)
        np.testing.assert_allclose(dZ[0, 0, c][:4, :4], Zfull[:4, :4], rtol=1e-14)


def test_groups_one_is_the_ungrouped_computation_bitwise():
    rng = np.random.default_rng(62)
    q, k, v = _rand(rng, 1, 9, 2, 8, 4)
    a = O.closed_form(q, k, v)
    b = O.closed_form(q, k, v, groups=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("g", [2, 4])
def test_grouped_backward_matches_central_finite_differences(g):
    rng = np.random.default_rng(70 + g)
    B, T, H, p, dv = 1, 6, 1, 8, 3
    q, k, v = _rand(rng, B, T, H, p, dv, unit_q=False)
    dO = rng.standard_normal((B, T, H, dv))
    eps = 1e-2
    dq, dk, dv_ = O.backward(q, k, v, dO, eps, block=4, groups=g)

    def loss(q, k, v):
        return float((O.closed_form(q, k, v, eps, groups=g)[0] * dO).sum())

    h = 1e-6
    for name, x, gr in (("q", q, dq), ("k", k, dk), ("v", v, dv_)):
        num = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**args_p) - loss(**args_m)) / (2 * h)
        np.testing.assert_allclose(gr, num, rtol=1e-6, atol=1e-7, err_msg=name)

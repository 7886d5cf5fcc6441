"""CPU fp64 oracle for causal, normalized linear attention with the rank-one PSD feature map.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the benchmark's
CPU-baseline leg may import this module.  It imports nothing from the GPU package, and the
GPU package never imports it; the two share no code.  It is slow on purpose: every function
is the plain definition (or the method's steps in the pages' order), written so that it can
be checked against the pages by eye.

Sources (page title, then section):
  [Gist]   "Technische Samenvatting" on gist.science, sections 2.1 (output gate), 2.2 (rank-one
           PSD features psi(u) = u u^T square the raw inner product), 2.3 (chunked
           parallelism, associative prefix scan over chunks, the two operating points).
  [AIsum]  "Kernelized Linear Attention ... AI summary" on ai.info, Main Findings: the bullet on
           the free readout gate (alpha_t = D_{t-1}/D_t, beta_t = c_t/D_t), the bullet on
           squaring the inner product, the bullet on state size (d^2 direct / d(d+1)/2 packed
           coordinates, feature-value state n*d_v), the bullet on the chunk recurrence.
  [Review] "Paper Review: Kernelized Linear Attention" on romaanj.github.io, Validation and
           Results paragraphs (exact O(T) chunked-state form; scan depth O(log(T/C))).
  [README] the KATA GitHub README (ayghri/KATA): the direct kernel call takes (B,T,H,D) tensors,
           and its usage example passes a factor count (num_groups) to the concatenated-PSD
           ("concat-SPD") kernel.
  KATA-Mg: [Gist 2.3] the variants bullet (several PSD factors); [AIsum state-size bullet]
           state d(d/g + 1)/2 * d_v, the full map at g = 1; [Review] Comparison paragraph
           (two 32-dimensional factors at head dimension 64, 135,168 state entries).

The computation (every array here is float64):
  feature(u)  = vec(u u^T), row-major index i*p + j                       [Gist 2.2]
  a[t,s]      = <feature(q_t), feature(k_s)> = (q_t . k_s)^2,  s <= t      [Gist 2.2; AIsum]
  D_t         = eps + sum_{s<=t} a[t,s]                                    [AIsum gate bullet]
  o_t         = sum_{s<=t} a[t,s] v_s / D_t                                [Gist 2.1; AIsum]
KATA-Mg (groups = g): the p coordinates form g consecutive groups of p/g; the feature is the
concatenation over groups of vec(u^(j) u^(j)^T), so a[t,s] = sum_j (q_t^(j) . k_s^(j))^2 with
one shared denominator.  groups = 1 is the computation above.
Readings where the pages are silent: eps is added once, outside the sum, eps = 1e-6; the
diagonal s = t is included (the gate's beta_t weights the current value v_t); no scaling or
normalization of q, k inside the operation; chunk c covers tokens [cC, (c+1)C) and T % C == 0.

Layout: public functions take (B, T, H, D) arrays, the layout of the pages' kernel call
[README]; heads are independent, and the per-head work is done on (T, D) slices.

Pins (each function is checked against something other than itself in tests/test_oracle.py):
  feature           integer identity <feature(q),feature(k)> == (q.k)^2; widths p^2 and
                    p(p+1)/2 printed for d = 64 [AIsum state-size bullet] (tests/golden).
  closed_form       textbook special cases (p = 1 weighted prefix mean, identical keys ->
                    causal running mean, orthonormal keys -> exact retrieval, q = 0 -> 0,
                    eps placement), invariants (nonnegative weights summing to 1 - eps/D_t,
                    convex hull, causality, permutation of the past), a hand-worked example.
  closed_form_rows  equals closed_form on every row it is asked for, plus the same cases.
  recurrent         the same special cases and invariants; equals closed_form.
  chunk_states      per-chunk sums checked against explicit outer-product sums.
  exclusive_scan    numpy.cumsum (library routine) and the defining invariants.
  chunked           C = T reduces to closed_form's single block, C = 1 to the recurrence,
                    equal to closed_form for every C dividing T; the special cases.
  gate_terms        alpha + beta == 1 and o_t == alpha_t * ohat_{t-1} + beta_t * v_t.
  backward          central finite differences of closed_form (fp64).
  groups (KATA-Mg)  groups = p reduces to the positive-orthant feature u*u (a closed form of
                    its own); every grouped output is the sum of per-group ungrouped numerators
                    over the sum of per-group denominators; integer identity for the grouped
                    feature; packed widths against the printed state sizes; every form agrees
                    with the grouped closed form; backward against finite differences.
"""

import numpy as np

__all__ = [
    "EPS",
    "feature",
    "closed_form",
    "closed_form_rows",
    "recurrent",
    "chunk_states",
    "exclusive_scan",
    "chunked",
    "gate_terms",
    "backward",
    "state_elems",
    "group_mask",
    "packed_width",
]

EPS = 1e-6


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _heads(x):
    """(B, T, H, D) -> iterator of (b, h, (T, D) view)."""
    B, _, H, _ = x.shape
    for b in range(B):
        for h in range(H):
            yield b, h, x[b, :, h, :]


def _group_slices(p, groups):
    if groups < 1 or p % groups:
        raise ValueError("groups must divide p")
    w = p // groups
    return [slice(j * w, (j + 1) * w) for j in range(groups)]


def feature(u, groups=1):
    """Rank-one PSD feature psi(u) = u u^T, flattened row-major: index i*p + j.

    [Gist 2.2] psi(u) = u u^T; [AIsum, squaring bullet] its inner product squares the raw
    inner product.  Works on any leading shape: (..., p) -> (..., p*p).
    groups = g (KATA-Mg [Gist 2.3 variants; README concat-SPD]): the concatenation over the g
    groups of consecutive coordinates of vec(u^(j) u^(j)^T), width p^2 / g.
    """
    u = _f64(u)
    p = u.shape[-1]
    if groups == 1:
        return (u[..., :, None] * u[..., None, :]).reshape(*u.shape[:-1], p * p)
    parts = [(u[..., sl, None] * u[..., None, sl]).reshape(*u.shape[:-1], -1)
             for sl in _group_slices(p, groups)]
    return np.concatenate(parts, axis=-1)


def group_mask(p, groups=1):
    """Boolean (p, p): True where coordinates i and j lie in the same group."""
    g = np.empty(p, dtype=np.int64)
    for j, sl in enumerate(_group_slices(p, groups)):
        g[sl] = j
    return g[:, None] == g[None, :]


def packed_width(p, groups=1):
    """Unique coordinates of the (grouped) feature: the pairs i <= j within one group,
    counted one by one.  [AIsum state-size bullet: d(d+1)/2 packed coordinates; KATA-Mg
    state d(d/g + 1)/2 * d_v.]"""
    m = group_mask(p, groups)
    return int(sum(1 for i in range(p) for j in range(i, p) if m[i, j]))


def _scores(Qb, Kb, groups):
    """a[t,s] = sum_j (q_t^(j) . k_s^(j))^2 for the rows of Qb against the rows of Kb."""
    a = 0.0
    for sl in _group_slices(Qb.shape[-1], groups):
        sc = Qb[:, sl] @ Kb[:, sl].T                  # q_t . k_s within one group
        a = a + sc * sc                               # (q_t . k_s)^2  [Gist 2.2]
    return a


def state_elems(p, dv):
    """Entries of one direct (unpacked) chunk state: S is p^2 x d_v plus the normalizer
    vec(Z) of length p^2, i.e. p^2 * (d_v + 1).  [AIsum state-size bullet: direct width d^2,
    feature-value state n * d_v.]"""
    return p * p * (dv + 1)


# ----------------------------------------------------------------------------------------
# Closed form (the definition), brute force over query blocks.
# ----------------------------------------------------------------------------------------

def _masked_sum(a, V, mask):
    """sum_s a[t,s] V[s] over the pairs where mask[t,s] holds, by selection: pairs outside
    the mask are never multiplied, so non-finite values there cannot leak in."""
    prod = np.where(mask[:, :, None], a[:, :, None] * V[None, :, :], 0.0)
    return prod.sum(axis=1)


def _closed_form_head(Q, K, V, eps, block, groups):
    T = Q.shape[0]
    o = np.empty((T, V.shape[1]))
    den = np.empty(T)
    for i0 in range(0, T, block):
        i1 = min(T, i0 + block)
        # keys before the block are in every row's past: plain products
        a = _scores(Q[i0:i1], K[:i0], groups)
        num = a @ V[:i0]
        asum = a.sum(axis=1)
        # keys inside the block: causal, diagonal included, by selection
        mask = np.arange(i0, i1)[None, :] <= np.arange(i0, i1)[:, None]
        ad = np.where(mask, _scores(Q[i0:i1], K[i0:i1], groups), 0.0)
        num = num + _masked_sum(ad, V[i0:i1], mask)
        d = eps + (asum + ad.sum(axis=1))             # D_t = eps + sum a  [AIsum gate]
        o[i0:i1] = num / d[:, None]                   # o_t = N_t / D_t    [Gist 2.1]
        den[i0:i1] = d
    return o, den


def closed_form(q, k, v, eps=EPS, block=512, groups=1):
    """o_t = sum_{s<=t} (q_t.k_s)^2 v_s / (eps + sum_{s<=t} (q_t.k_s)^2), per (b, h).

    Inputs (B,T,H,p), (B,T,H,p), (B,T,H,d_v); returns (o (B,T,H,d_v), D (B,T,H)), float64.
    Brute force over query blocks of `block` rows; masked pairs are selected away, never
    multiplied by zero, so a non-finite value in a future token cannot reach o_t.
    groups = g: the KATA-Mg score sum_j (q_t^(j) . k_s^(j))^2.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, _ = q.shape
    o = np.empty((B, T, H, v.shape[-1]))
    den = np.empty((B, T, H))
    for b, h, Q in _heads(q):
        o[b, :, h], den[b, :, h] = _closed_form_head(Q, k[b, :, h], v[b, :, h], eps, block,
                                                     groups)
    return o, den


def closed_form_rows(q, k, v, rows, eps=EPS, block=256, groups=1):
    """The closed form for selected rows of ONE head.

    q, k: (T, p); v: (T, d_v); rows: 1-D int array of token indices.  Returns
    (o (len(rows), d_v), D (len(rows),)) in the order given.  Each row t uses keys s <= t
    only; rows are grouped in blocks to use matrix products.
    """
    Q, K, V = _f64(q), _f64(k), _f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    order = np.argsort(rows, kind="stable")
    o = np.empty((rows.size, V.shape[1]))
    den = np.empty(rows.size)
    for j0 in range(0, rows.size, block):
        sel = order[j0:j0 + block]
        t = rows[sel]
        s0 = int(t.min())                             # keys < s0 are past for every row
        a = _scores(Q[t], K[:s0], groups)
        num = a @ V[:s0]
        asum = a.sum(axis=1)
        for r, tr in enumerate(t):                    # the rest: keys s0..t of this row only
            at = _scores(Q[tr:tr + 1], K[s0:tr + 1], groups)[0]
            num[r] += at @ V[s0:tr + 1]
            asum[r] += at.sum()
        d = eps + asum
        o[sel] = num / d[:, None]
        den[sel] = d
    return o, den


# ----------------------------------------------------------------------------------------
# Recurrent form: the fixed-size state updated token by token.
# ----------------------------------------------------------------------------------------

def recurrent(q, k, v, eps=EPS, groups=1):
    """S_t = S_{t-1} + feature(k_t) v_t^T,  Z_t = Z_{t-1} + k_t k_t^T,
    o_t = S_t^T feature(q_t) / (eps + q_t^T Z_t q_t).

    [Gist 2.3 / AIsum: linear attention as a recurrence on a fixed-size state; the update is
    additive and commutative].  Token-by-token Python loop: small inputs only.  groups = g:
    the grouped feature, and Z keeps only its within-group entries.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, p = q.shape
    dv = v.shape[-1]
    gm = group_mask(p, groups)
    o = np.empty((B, T, H, dv))
    den = np.empty((B, T, H))
    for b, h, Q in _heads(q):
        K, V = k[b, :, h], v[b, :, h]
        S = np.zeros((p * p // groups, dv))
        Z = np.zeros((p, p))
        for t in range(T):
            S += np.outer(feature(K[t], groups), V[t])
            Z += np.where(gm, np.outer(K[t], K[t]), 0.0)
            d = eps + Q[t] @ Z @ Q[t]
            o[b, t, h] = feature(Q[t], groups) @ S / d
            den[b, t, h] = d
    return o, den


# ----------------------------------------------------------------------------------------
# Chunked-state form: per-chunk states, exclusive prefix scan, intra-chunk block.
# ----------------------------------------------------------------------------------------

def chunk_states(k, v, C, groups=1):
    """Per-chunk states of every head.

    dS_c = sum_{s in chunk c} feature(k_s) v_s^T   (p^2 x d_v)
    dZ_c = sum_{s in chunk c} k_s k_s^T            (p x p)
    [Gist 2.3: chunked parallelism; AIsum chunk-recurrence bullet: inter-chunk cost
    O(C n_psi d_v)].  Returns dS (B,H,Nc,p*p,d_v) and dZ (B,H,Nc,p,p).  groups = g: the
    grouped feature (p^2/g rows) and the within-group entries of dZ.
    """
    k, v = _f64(k), _f64(v)
    B, T, H, p = k.shape
    dv = v.shape[-1]
    if T % C:
        raise ValueError("T must be a multiple of the chunk size")
    nc = T // C
    gm = group_mask(p, groups)
    dS = np.empty((B, H, nc, p * p // groups, dv))
    dZ = np.empty((B, H, nc, p, p))
    for b, h, K in _heads(k):
        V = v[b, :, h]
        for c in range(nc):
            Kc, Vc = K[c * C:(c + 1) * C], V[c * C:(c + 1) * C]
            dS[b, h, c] = feature(Kc, groups).T @ Vc
            dZ[b, h, c] = np.where(gm, Kc.T @ Kc, 0.0)
    return dS, dZ


def exclusive_scan(x, axis=2):
    """Exclusive prefix sum along `axis`: out[c] = sum_{i<c} x[i], out[0] = 0; also returns
    the inclusive total sum_i x[i].

    [Gist 2.3: inter-chunk state propagation is an associative scan (parallel prefix sum);
    AIsum: the update is additive, so the associative operator is plain addition.]  Written
    as the sequential definition; its parallel (tree) evaluation gives the same sums.
    """
    x = np.moveaxis(_f64(x), axis, 0)
    out = np.empty_like(x)
    run = np.zeros_like(x[0])
    for c in range(x.shape[0]):
        out[c] = run
        run = run + x[c]
    return np.moveaxis(out, 0, axis), run


def chunked(q, k, v, C, eps=EPS, groups=1):
    """Exact O(T) chunked-state form.  For t in chunk c:

    num_t = feature(q_t)^T S_{<c} + sum_{s in c, s<=t} a[t,s] v_s
    D_t   = eps + q_t^T Z_{<c} q_t + sum_{s in c, s<=t} a[t,s]
    o_t   = num_t / D_t

    with S_{<c}, Z_{<c} the exclusive prefix scan of the chunk states.  [Gist 2.3: intra-chunk
    attention is a dense tile, inter-chunk propagation a prefix scan; Review: the chunked form
    is exact.]  Returns (o, D) like closed_form.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, p = q.shape
    dv = v.shape[-1]
    dS, dZ = chunk_states(k, v, C, groups)
    S_prev, _ = exclusive_scan(dS, axis=2)
    Z_prev, _ = exclusive_scan(dZ, axis=2)
    o = np.empty((B, T, H, dv))
    den = np.empty((B, T, H))
    tri = np.tril(np.ones((C, C), dtype=bool))
    for b, h, Q in _heads(q):
        K, V = k[b, :, h], v[b, :, h]
        for c in range(T // C):
            sl = slice(c * C, (c + 1) * C)
            Qc, Kc, Vc = Q[sl], K[sl], V[sl]
            inter_num = feature(Qc, groups) @ S_prev[b, h, c]
            inter_den = np.einsum("ti,ij,tj->t", Qc, Z_prev[b, h, c], Qc)
            a = np.where(tri, _scores(Qc, Kc, groups), 0.0)
            d = eps + inter_den + a.sum(axis=1)
            o[b, sl, h] = (inter_num + _masked_sum(a, Vc, tri)) / d[:, None]
            den[b, sl, h] = d
    return o, den


# ----------------------------------------------------------------------------------------
# The convex output gate.
# ----------------------------------------------------------------------------------------

def gate_terms(q, k, v, eps=EPS):
    """alpha_t, beta_t and the previous readout ohat_{t-1}, all read with the query q_t.

    [AIsum gate bullet; Gist 2.1] With D_{t-1}(q_t) = eps + sum_{s<t} a[t,s], c_t = a[t,t],
    D_t = D_{t-1} + c_t:  alpha_t = D_{t-1}/D_t, beta_t = c_t/D_t, and
    ohat_{t-1} = sum_{s<t} a[t,s] v_s / D_{t-1} (zero at t = 0, where D_{-1} = eps).
    Then o_t = alpha_t ohat_{t-1} + beta_t v_t.  Returns arrays shaped (B,T,H), (B,T,H),
    (B,T,H,d_v).  Brute force, small inputs.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, _ = q.shape
    alpha = np.empty((B, T, H))
    beta = np.empty((B, T, H))
    ohat = np.empty((B, T, H, v.shape[-1]))
    for b, h, Q in _heads(q):
        K, V = k[b, :, h], v[b, :, h]
        for t in range(T):
            past = (K[:t] @ Q[t]) ** 2                 # a[t, s], s < t
            cur = (K[t] @ Q[t]) ** 2                   # c_t = a[t, t]
            d_prev = eps + past.sum()
            d_now = d_prev + cur
            alpha[b, t, h] = d_prev / d_now
            beta[b, t, h] = cur / d_now
            ohat[b, t, h] = (past @ V[:t]) / d_prev
    return alpha, beta, ohat


# ----------------------------------------------------------------------------------------
# Backward of the closed form.
# ----------------------------------------------------------------------------------------

def backward(q, k, v, dO, eps=EPS, block=512, groups=1):
    """Gradients of L = sum_t <dO_t, o_t> with o the closed form (derived here; the pages
    name a flash backward [README kernel list] but print no formula).

    Per head, with s_ts = q_t . k_s and a_ts = s_ts^2 for s <= t:
      delta_t = dO_t . o_t
      G_ts    = (dO_t . v_s - delta_t) / D_t                (s <= t)
      dq_t    = sum_s 2 s_ts G_ts k_s
      dk_s    = sum_t 2 s_ts G_ts q_t
      dv_s    = sum_{t>=s} a_ts dO_t / D_t
    Tiled over query blocks; returns float64 (dq, dk, dv).  groups = g: a_ts is the grouped
    score, and the coordinates of group j take s_ts^(j) = q_t^(j) . k_s^(j) in place of s_ts.
    """
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    T, p = q.shape[1], q.shape[3]
    slices = _group_slices(p, groups)
    for b, h, Q in _heads(q):
        K, V, G_out = k[b, :, h], v[b, :, h], dO[b, :, h]
        for i0 in range(0, T, block):
            i1 = min(T, i0 + block)
            t_idx = np.arange(i0, i1)[:, None]
            mask = np.arange(i1)[None, :] <= t_idx
            scs = [np.where(mask, Q[i0:i1, sl] @ K[:i1, sl].T, 0.0) for sl in slices]
            a = sum(sc * sc for sc in scs)
            d = eps + a.sum(axis=1)
            o = (a @ V[:i1]) / d[:, None]
            dOb = G_out[i0:i1]
            delta = (dOb * o).sum(axis=1)
            g = np.where(mask, (dOb @ V[:i1].T - delta[:, None]) / d[:, None], 0.0)
            for sl, sc in zip(slices, scs):
                ds = 2.0 * sc * g
                dq[b, i0:i1, h, sl] = ds @ K[:i1, sl]
                dk[b, :i1, h, sl] += ds.T @ Q[i0:i1, sl]
            dv[b, :i1, h] += (a / d[:, None]).T @ dOb
    return dq, dk, dv

"""Plants plausible mistakes in a scratch copy of the CPU oracle and checks that the oracle's
pins (tests/test_oracle.py) catch every one: a dropped eps, an excluded diagonal, |q.k|
instead of (q.k)^2, a state read before its update, an inclusive scan, a wrong sign or a
perturbed operand in the backward, a shifted feature index, a wrong gate weight, and KATA-Mg
grouping mistakes that leave the ungrouped computation unchanged.  CPU only."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kata_oracle.py")

MUTATIONS = {
    "drop_eps": ("d = eps + (asum + ad.sum(axis=1))", "d = (asum + ad.sum(axis=1))"),
    "exclude_diagonal": (
        "mask = np.arange(i0, i1)[None, :] <= np.arange(i0, i1)[:, None]",
        "mask = np.arange(i0, i1)[None, :] < np.arange(i0, i1)[:, None]"),
    "abs_instead_of_square": (
        "a = a + sc * sc                               # (q_t . k_s)^2  [Gist 2.2]",
        "a = a + np.abs(sc)"),
    # KATA-Mg: each of these is invisible at groups = 1
    "groups_square_of_sum": (
        "        a = a + sc * sc                               # (q_t . k_s)^2  [Gist 2.2]\n"
        "    return a",
        "        a = a + sc\n    return a * a"),
    "groups_recurrent_full_Z": ("Z += np.where(gm, np.outer(K[t], K[t]), 0.0)",
                                "Z += np.outer(K[t], K[t])"),
    "groups_chunk_full_Z": ("dZ[b, h, c] = np.where(gm, Kc.T @ Kc, 0.0)",
                            "dZ[b, h, c] = Kc.T @ Kc"),
    "groups_backward_wrong_slice": ("dq[b, i0:i1, h, sl] = ds @ K[:i1, sl]",
                                    "dq[b, i0:i1, h, sl] = ds @ K[:i1, slices[0]]"),
    "rows_skip_diagonal": (
        "at = _scores(Q[tr:tr + 1], K[s0:tr + 1], groups)[0]\n"
        "            num[r] += at @ V[s0:tr + 1]",
        "at = _scores(Q[tr:tr + 1], K[s0:tr], groups)[0]\n"
        "            num[r] += at @ V[s0:tr]"),
    "recurrent_eps_squared": ("d = eps + Q[t] @ Z @ Q[t]", "d = eps * eps + Q[t] @ Z @ Q[t]"),
    "recurrent_read_before_update": (
        "            S += np.outer(feature(K[t], groups), V[t])\n"
        "            Z += np.where(gm, np.outer(K[t], K[t]), 0.0)\n"
        "            d = eps + Q[t] @ Z @ Q[t]\n"
        "            o[b, t, h] = feature(Q[t], groups) @ S / d",
        "            d = eps + Q[t] @ Z @ Q[t]\n"
        "            o[b, t, h] = feature(Q[t], groups) @ S / d\n"
        "            S += np.outer(feature(K[t], groups), V[t])\n"
        "            Z += np.where(gm, np.outer(K[t], K[t]), 0.0)"),
    "inclusive_scan": ("        out[c] = run\n        run = run + x[c]",
                       "        run = run + x[c]\n        out[c] = run"),
    "chunk_denominator_operand": (
        'inter_den = np.einsum("ti,ij,tj->t", Qc, Z_prev[b, h, c], Qc)',
        'inter_den = np.einsum("ti,ij,tj->t", Qc, Z_prev[b, h, c], Qc * 0 + 1)'),
    "backward_delta_sign": (
        "g = np.where(mask, (dOb @ V[:i1].T - delta[:, None]) / d[:, None], 0.0)",
        "g = np.where(mask, (dOb @ V[:i1].T + delta[:, None]) / d[:, None], 0.0)"),
    "backward_dk_scaled": ("dk[b, :i1, h, sl] += ds.T @ Q[i0:i1, sl]",
                           "dk[b, :i1, h, sl] += 1.0001 * (ds.T @ Q[i0:i1, sl])"),
    "feature_shifted_index": (
        "return (u[..., :, None] * u[..., None, :]).reshape(*u.shape[:-1], p * p)",
        "return (u[..., :, None] * np.roll(u, 1, axis=-1)[..., None, :])"
        ".reshape(*u.shape[:-1], p * p)"),
    "gate_beta_denominator": ("beta[b, t, h] = cur / d_now", "beta[b, t, h] = cur / d_prev"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, "mutation site not found: the oracle changed; update the site"
    (tmp_path / "oracle").mkdir()
    (tmp_path / "tests").mkdir()
    (tmp_path / "oracle" / "kata_oracle.py").write_text(src.replace(old, new))
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), tmp_path / "oracle")
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    for f in ("test_oracle.py", "conftest.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 1, f"planted mistake {name!r} passed every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout

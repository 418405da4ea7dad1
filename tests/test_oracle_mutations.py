"""The oracle's pins must catch plausible mistakes.

Each case below plants one slip into a private copy of the oracle's source (on
the CPU, never in the real module) and checks that the independent pins --
numpy's covariance, the unrolled GLA / Gated DeltaNet sums, the hand-derived
fixtures and the gate formula -- reject the mutant.
"""

import json
import os
import types

import numpy as np
import pytest
from scipy.special import expit

from curvature_conditioned_query_amd.inputs import gdn_inputs, gla_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ccq.py")
GOLDEN = os.path.join(ROOT, "tests", "golden", "hand_cases.json")

MUTATIONS = {
    "dropped_mu_mu_T": ("Sigma = Cbar - mu[..., :, None] * mu[..., None, :]", "Sigma = Cbar"),
    "ddof_one": ("Cbar = st.C / nn[..., None, None]", "Cbar = st.C / np.maximum(nn - 1, 1)[..., None, None]"),
    "cleaning_sign": ("q_clean = qt - lam[..., None]", "q_clean = qt + lam[..., None]"),
    "gate_on_key": ('np.einsum("bhd,hd->bh", qt, w_lam)', 'np.einsum("bhd,hd->bh", kt, w_lam)'),
    "gla_decay_on_value_side": ("st.S * np.exp(g[:, :, t])[..., None, :]", "st.S * np.exp(g[:, :, t])[..., :, None]"),
    "gdn_no_alpha_on_state": ("st.S = a * (st.S - bt * Sk * kt[..., None, :])", "st.S = (st.S - bt * Sk * kt[..., None, :])"),
    "read_raw_query": ("np.matmul(st.S, q_clean[..., None])", "np.matmul(st.S, qt[..., None])"),
    "decayed_statistics": ("st.C = st.C + kt[..., :, None] * kt[..., None, :]",
                           "st.C = 0.9 * st.C + kt[..., :, None] * kt[..., None, :]"),
    "stats_skip_current_token": ("st.C = st.C + kt[..., :, None] * kt[..., None, :]\n        st.m = st.m + kt",
                                 "pass"),
    "packed_lower_triangle": ("    iu, ju = np.triu_indices(d)\n    return C[..., iu, ju]",
                              "    iu, ju = np.tril_indices(d)\n    return C[..., iu, ju]"),
}


def _mutant(name):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _pins_hold(m) -> bool:
    """A compact run of independent pins against module m; False if any fails."""
    try:
        # covariance vs numpy (ddof 0, token t included)
        rng = np.random.default_rng(0)
        K = rng.standard_normal((6, 4))
        K /= np.linalg.norm(K, axis=1, keepdims=True)
        z = np.zeros((1, 1, 6, 4))
        _, _, rec = m.ccq_recurrent(z, K[None, None], np.zeros((1, 1, 6, 1)), z, None, np.zeros((1, 4)),
                                    np.zeros(1), "gla", record=True, record_sigma=True)
        for t in range(1, 7):
            if not np.allclose(rec["sigma"][0, 0, t - 1], np.cov(K[:t].T, bias=True), atol=1e-12):
                return False
        # packed statistic: the upper triangle row by row (hand case; C is symmetric, so the
        # lower triangle row by row would give 1 2 4 3 5 6)
        C3 = np.array([[1.0, 2.0, 3.0], [2.0, 4.0, 5.0], [3.0, 5.0, 6.0]])
        if not np.array_equal(m.pack_upper(C3), [1.0, 2.0, 3.0, 4.0, 5.0, 6.0]):
            return False
        # gate formula on the raw query
        x = gla_inputs(1, 1, 5, 4, 3, "f32")
        _, _, rec = m.ccq_recurrent(x.q, x.k, x.v, x.g, None, x.w_lam, x.b_lam, "gla", record=True)
        lam = expit(x.q[0, 0].astype(float) @ x.w_lam[0].astype(float) + x.b_lam[0])
        if not np.allclose(rec["lam"][0, 0], lam, rtol=1e-12):
            return False
        # hand-derived fixtures
        for c in json.load(open(GOLDEN))["cases"]:
            arr = lambda key: np.asarray(c[key], dtype=float)[None, None]  # noqa: E731
            beta = None if c["beta"] is None else arr("beta")
            o, _ = m.ccq_recurrent(arr("q"), arr("k"), arr("v"), arr("g"), beta, np.asarray(c["w"], float),
                                   np.asarray(c["b"], float), c["rule"])
            if not np.allclose(o[0, 0], np.asarray(c["o"]), atol=1e-12):
                return False
        # unrolled GLA with the cleaning off
        x = gla_inputs(1, 1, 8, 4, 5, "f32")
        x.b_lam[:] = -np.inf
        o, _ = m.ccq_recurrent(x.q, x.k, x.v, x.g, None, x.w_lam, x.b_lam, "gla")
        q, k, v, g = (a[0, 0].astype(float) for a in (x.q, x.k, x.v, x.g))
        ref = np.zeros((8, 4))
        for t in range(8):
            for j in range(t + 1):
                ref[t] += v[j] * np.sum(q[t] * k[j] * np.exp(g[j + 1:t + 1].sum(axis=0)))
        if not np.allclose(o[0, 0], ref, atol=1e-12):
            return False
        # unrolled Gated DeltaNet state
        x = gdn_inputs(1, 1, 6, 4, 7, "f32")
        _, st = m.ccq_recurrent(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, "gdn")
        k, v = x.k[0, 0].astype(float), x.v[0, 0].astype(float)
        a, b = np.exp(x.g[0, 0].astype(float)), x.beta[0, 0].astype(float)
        S = np.zeros((4, 4))
        for j in range(6):
            M = b[j] * np.outer(v[j], k[j])
            for jj in range(j + 1, 6):
                M = M @ (a[jj] * (np.eye(4) - b[jj] * np.outer(k[jj], k[jj])))
            S += M
        return bool(np.allclose(st.S[0, 0], S, atol=1e-12))
    except Exception:
        return False


def test_unmutated_oracle_passes_compact_pins():
    import oracle.ccq as real
    assert _pins_hold(real)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    assert not _pins_hold(_mutant(name)), f"pins did not catch mutation {name}"

"""Pins of the fp64 oracle against things other than itself.

Each test ties one part of ``oracle`` to a closed form, a brute-force
evaluation, a library routine, an invariant the pages state, or a hand-derived
fixture (``tests/golden/hand_cases.json``).  Together they are chosen so that a
plausible slip (a dropped mu mu^T term, 1/(t-1) instead of 1/t, statistics that
skip token t, a read before the write, a decay on the wrong side, a flipped
sign of the cleaning term, the wrong gate input) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

from curvature_conditioned_query_amd.inputs import (bf16_bits, bf16_round, gdn_inputs, gla_inputs,
                                                    structured_inputs)
from oracle import (Carry, ccq_chunked, ccq_decode_step, ccq_recurrent, gla_closed_form_carry,
                    key_covariance, normwise_error, pack_upper, unit_keys, unpack_upper)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _unit(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _run(x, **kw):
    return ccq_recurrent(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, x.rule, **kw)


def _sigmas(K, rule="gla"):
    """Sigma_t recorded by the recurrent oracle for a single chain of keys K [T, d]."""
    T, d = K.shape
    q = np.zeros((1, 1, T, d))
    v = np.zeros((1, 1, T, 1))
    g = np.zeros((1, 1, T, d))
    _, _, rec = ccq_recurrent(q, K[None, None], v, g, None, np.zeros((1, d)), np.zeros(1), "gla",
                              record=True, record_sigma=True)
    return rec["sigma"][0, 0]


# ---------------------------------------------------------------- Sigma_t


def test_sigma_is_hessian_of_log_partition():
    """Sigma_t is the Hessian at q = 0 of A_t(q) = log sum_{j<=t} exp(k_j . q), and the
    gradient there is mu_t (summary §2 "理论推导"; write-up "方法解析").  Checked by central
    finite differences of the log-partition itself."""
    rng = np.random.default_rng(11)
    d, T = 5, 7
    K = _unit(rng, T, d)
    sig = _sigmas(K)
    h = 1e-4
    eye = np.eye(d)
    for t in (1, 3, 7):
        Kt = K[:t]

        def A(qv):
            z = Kt @ qv
            return float(np.log(np.sum(np.exp(z))))

        Hfd = np.zeros((d, d))
        for a in range(d):
            for b in range(d):
                ea, eb = h * eye[a], h * eye[b]
                Hfd[a, b] = (A(ea + eb) - A(ea - eb) - A(-ea + eb) + A(-ea - eb)) / (4 * h * h)
        np.testing.assert_allclose(sig[t - 1], Hfd, atol=2e-7)
        grad = np.array([(A(h * eye[a]) - A(-h * eye[a])) / (2 * h) for a in range(d)])
        np.testing.assert_allclose(grad, Kt.mean(axis=0), atol=1e-8)


@pytest.mark.parametrize("d", [2, 5, 8])
def test_sigma_matches_population_covariance(d):
    """Sigma_t equals numpy's covariance with ddof = 0 over keys j <= t (token t included)."""
    rng = np.random.default_rng(d)
    K = _unit(rng, 8, d)
    sig = _sigmas(K)
    for t in range(1, 9):
        ref = np.cov(K[:t].T, bias=True).reshape(d, d)
        np.testing.assert_allclose(sig[t - 1], ref, atol=1e-14)
        np.testing.assert_allclose(key_covariance(K[:t]), ref, atol=1e-14)


def test_sigma_special_cases():
    """t = 1 gives Sigma = 0 (so q_clean = q exactly); identical keys give 0; orthonormal keys
    e_1..e_t give (1/t) P_t - (1/t^2) 1 1^T with eigenvalues 1/t (t - 1 times) and 0."""
    rng = np.random.default_rng(3)
    d = 6
    # t = 1
    x = gla_inputs(2, 3, 1, d, 5, "f32")
    _, _, rec = _run(x, record=True, record_sigma=True)
    assert np.all(rec["sigma"] == 0.0)
    assert np.array_equal(rec["q_clean"], x.q.astype(np.float64))
    # identical keys
    k = _unit(rng, 1, d)
    sig = _sigmas(np.repeat(k, 9, axis=0))
    assert np.max(np.abs(sig)) < 1e-15
    # orthonormal keys
    sig = _sigmas(np.eye(d)[:5])
    for t in range(1, 6):
        ref = np.zeros((d, d))
        ref[:t, :t] = np.eye(t) / t - np.ones((t, t)) / t ** 2
        np.testing.assert_allclose(sig[t - 1], ref, atol=1e-15)
        ev = np.sort(np.linalg.eigvalsh(sig[t - 1]))
        expect = np.sort(np.r_[np.full(t - 1, 1.0 / t), np.zeros(d - t + 1)])
        np.testing.assert_allclose(ev, expect, atol=1e-14)


def test_eigenvalue_bound_for_unit_keys():
    """With unit keys, Sigma is PSD with trace 1 - |mu|^2 <= 1, so the cleaning operator
    I - lambda Sigma has its spectrum in [1 - lambda, 1] (write-up "方法解析", point 2)."""
    rng = np.random.default_rng(7)
    for d in (3, 16):
        K = _unit(rng, 40, d)
        sig = _sigmas(K)
        for t in (1, 2, 5, 40):
            mu = K[:t].mean(axis=0)
            assert abs(np.trace(sig[t - 1]) - (1 - mu @ mu)) < 1e-13
            for lam in (0.05, 0.5, 1.0):
                ev = np.linalg.eigvalsh(np.eye(d) - lam * sig[t - 1])
                assert ev.min() >= 1 - lam - 1e-13 and ev.max() <= 1 + 1e-13
                assert ev.min() >= 1 - lam * (1 - mu @ mu) - 1e-13


def test_correction_score_is_a_covariance():
    """k_j^T Sigma_t q equals the population covariance over i <= t of (k_j . k_i, k_i . q)
    (write-up "方法解析")."""
    rng = np.random.default_rng(5)
    d, t = 7, 12
    K = _unit(rng, t, d)
    q = rng.standard_normal(d)
    sig = _sigmas(K)[t - 1]
    for j in (0, 4, 11):
        ref = np.cov(np.stack([K @ K[j], K @ q]), bias=True)[0, 1]
        assert abs(K[j] @ sig @ q - ref) < 1e-14


# ---------------------------------------------------------------- gate and cleaning


def test_gate_and_cleaned_query():
    """lambda_t = sigmoid(w . q_t + b) on the raw query, and q_clean = q - lambda grad_q(q^T Sigma q / 2),
    the gradient taken by finite differences with Sigma from numpy's covariance."""
    x = gla_inputs(1, 2, 9, 6, 21, "f32")
    _, _, rec = _run(x, record=True)
    q = x.q.astype(np.float64)
    lam_ref = expit(np.einsum("bhtd,hd->bht", q, x.w_lam.astype(np.float64)) + x.b_lam[None, :, None])
    np.testing.assert_allclose(rec["lam"], lam_ref, rtol=1e-14)
    h = 1e-5
    for hh in range(2):
        K = x.k[0, hh].astype(np.float64)
        for t in (1, 4, 9):
            Sig = np.cov(K[:t].T, bias=True)
            qt = q[0, hh, t - 1]
            f = lambda z: 0.5 * z @ Sig @ z  # noqa: E731
            grad = np.array([(f(qt + h * e) - f(qt - h * e)) / (2 * h) for e in np.eye(6)])
            ref = qt - lam_ref[0, hh, t - 1] * grad
            np.testing.assert_allclose(rec["q_clean"][0, hh, t - 1], ref, atol=1e-9)


def test_fixed_lambda_gate():
    """w = 0 and b = logit(lambda) give q_clean = (I - lambda Sigma) q exactly (the fixed
    lambda = 0.1 variant of the write-up's gate ablation)."""
    x = gla_inputs(1, 1, 10, 5, 9, "f32")
    lam = 0.1
    x.w_lam[:] = 0
    x.b_lam[:] = math.log(lam / (1 - lam))
    _, _, rec = _run(x, record=True)
    K = x.k[0, 0].astype(np.float64)
    for t in range(1, 11):
        Sig = np.cov(K[:t].T, bias=True)
        ref = (np.eye(5) - lam * Sig) @ x.q[0, 0, t - 1].astype(np.float64)
        np.testing.assert_allclose(rec["q_clean"][0, 0, t - 1], ref, atol=1e-15)


# ---------------------------------------------------------------- backbones


def test_lambda_zero_gla_is_unrolled_gla():
    """b = -inf switches the cleaning off exactly; then o_t must equal the O(T^2) unrolled GLA
    sum o_t = sum_{j<=t} v_j sum_c q_tc k_jc exp(sum_{j<j'<=t} g_j'c)."""
    x = gla_inputs(1, 2, 11, 4, 31, "f32")
    x.b_lam[:] = -np.inf
    o, _ = _run(x)
    q, k, v, g = (a.astype(np.float64) for a in (x.q, x.k, x.v, x.g))
    ref = np.zeros_like(o)
    for hh in range(2):
        for t in range(11):
            for j in range(t + 1):
                decay = np.exp(g[0, hh, j + 1:t + 1].sum(axis=0))
                ref[0, hh, t] += v[0, hh, j] * np.sum(q[0, hh, t] * k[0, hh, j] * decay)
    np.testing.assert_allclose(o, ref, atol=1e-13)


def test_no_decay_no_gate_is_linear_attention():
    """g = 0 and lambda = 0: plain linear attention o_t = sum_{j<=t} v_j (k_j . q_t)."""
    x = gla_inputs(2, 1, 13, 5, 41, "f32")
    x.b_lam[:] = -np.inf
    x.g[:] = 0
    o, _ = _run(x)
    q, k, v = (a.astype(np.float64) for a in (x.q, x.k, x.v))
    scores = np.tril(np.einsum("bhtd,bhjd->bhtj", q, k))
    np.testing.assert_allclose(o, scores @ v, atol=1e-13)


def test_gdn_unrolled_products():
    """Gated DeltaNet state after T tokens equals the unrolled sum
    S_T = sum_j beta_j v_j k_j^T prod_{j<j'<=T} alpha_j' (I - beta_j' k_j' k_j'^T)."""
    x = gdn_inputs(1, 1, 7, 4, 51, "f32")
    _, st = _run(x)
    k, v = x.k[0, 0].astype(np.float64), x.v[0, 0].astype(np.float64)
    a = np.exp(x.g[0, 0].astype(np.float64))
    b = x.beta[0, 0].astype(np.float64)
    S = np.zeros((4, 4))
    for j in range(7):
        M = b[j] * np.outer(v[j], k[j])
        for jj in range(j + 1, 7):
            M = M @ (a[jj] * (np.eye(4) - b[jj] * np.outer(k[jj], k[jj])))
        S += M
    np.testing.assert_allclose(st.S[0, 0], S, atol=1e-14)


def test_gdn_beta_one_retrieves_last_value():
    """Delta rule with beta = 1 and a unit key stores v_t exactly along k_t: S_t k_t = v_t."""
    x = gdn_inputs(1, 1, 9, 6, 61, "f32")
    x.beta[:] = 1.0
    for t in range(1, 10):
        _, st = ccq_recurrent(x.q[:, :, :t], x.k[:, :, :t], x.v[:, :, :t], x.g[:, :, :t], x.beta[:, :, :t],
                              x.w_lam, x.b_lam, "gdn")
        np.testing.assert_allclose(st.S[0, 0] @ x.k[0, 0, t - 1].astype(np.float64),
                                   x.v[0, 0, t - 1].astype(np.float64), atol=2e-6)


def test_gdn_orthonormal_keys_do_not_interfere():
    """With orthonormal keys the delta term vanishes: S_T k_j = beta_j v_j prod_{j'>j} alpha_j'."""
    x = gdn_inputs(1, 1, 5, 5, 71, "f32")
    x.k[0, 0] = np.eye(5, dtype=np.float32)
    _, st = _run(x)
    a = np.exp(x.g[0, 0].astype(np.float64))
    for j in range(5):
        ref = x.beta[0, 0, j] * x.v[0, 0, j].astype(np.float64) * np.prod(a[j + 1:])
        np.testing.assert_allclose(st.S[0, 0] @ np.eye(5)[j], ref, atol=1e-15)


def test_hand_derived_fixtures():
    """Small cases worked out by hand (tests/golden/hand_cases.json)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        arr = lambda key: np.asarray(c[key], dtype=np.float64)[None, None]  # noqa: E731
        beta = None if c["beta"] is None else arr("beta")
        o, st, rec = ccq_recurrent(arr("q"), arr("k"), arr("v"), arr("g"), beta, np.asarray(c["w"], float),
                                   np.asarray(c["b"], float), c["rule"], record=True, record_sigma=True)
        np.testing.assert_allclose(o[0, 0], np.asarray(c["o"]), atol=1e-12, err_msg=c["name"])
        if "sigma_2" in c:
            np.testing.assert_allclose(rec["sigma"][0, 0, 1], np.asarray(c["sigma_2"]), atol=1e-15)
        if "S_2" in c:
            np.testing.assert_allclose(st.S[0, 0], np.asarray(c["S_2"]), atol=1e-15)


# ---------------------------------------------------------------- chunked algebra, carry, decode


@pytest.mark.parametrize("rule", ["gla", "gdn"])
@pytest.mark.parametrize("chunk", [1, 8, 16, 64])
def test_chunked_equals_recurrent(rule, chunk):
    """The chunk algebra reaches the per-token result for any chunk size and a ragged T."""
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(2, 2, 150, 12, 81, "f32")
    o1, c1 = _run(x)
    o2, c2 = ccq_chunked(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule, chunk=chunk)
    assert normwise_error(o2, o1) < 1e-12
    for a, b in ((c2.S, c1.S), (c2.C, c1.C), (c2.m, c1.m)):
        assert normwise_error(a, b) < 1e-12
    assert np.array_equal(c2.n, c1.n)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_chunked_structured_keys(rule):
    x = structured_inputs(rule, 1, 2, 200, 16, 91, "f32")
    o1, _ = _run(x)
    o2, _ = ccq_chunked(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule)
    assert normwise_error(o2, o1) < 1e-12


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_carry_split_and_resume(rule):
    """prefill(T1) then prefill(T2) from its carry equals prefill(T1 + T2)."""
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(1, 2, 90, 8, 101, "f32")
    o, st = _run(x)
    a, b = x.slab(0, 0), None  # noqa: F841
    sl1 = lambda arr: None if arr is None else arr[:, :, :37]  # noqa: E731
    sl2 = lambda arr: None if arr is None else arr[:, :, 37:]  # noqa: E731
    o1, c1 = ccq_recurrent(sl1(x.q), sl1(x.k), sl1(x.v), sl1(x.g), sl1(x.beta), x.w_lam, x.b_lam, rule)
    o2, c2 = ccq_chunked(sl2(x.q), sl2(x.k), sl2(x.v), sl2(x.g), sl2(x.beta), x.w_lam, x.b_lam, rule, carry=c1)
    assert normwise_error(np.concatenate([o1, o2], axis=2), o) < 1e-12
    assert normwise_error(c2.S, st.S) < 1e-12 and normwise_error(c2.C, st.C) < 1e-12
    assert np.array_equal(c2.n, st.n)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_decode_continues_prefill(rule):
    """prefill(T) then one decode step equals row T + 1 of prefill(T + 1)."""
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(3, 2, 41, 8, 111, "f32")
    o, st = _run(x)
    pre = lambda arr: None if arr is None else arr[:, :, :40]  # noqa: E731
    last = lambda arr: None if arr is None else arr[:, :, 40]  # noqa: E731
    _, c = ccq_recurrent(pre(x.q), pre(x.k), pre(x.v), pre(x.g), pre(x.beta), x.w_lam, x.b_lam, rule)
    od, cd = ccq_decode_step(last(x.q), last(x.k), last(x.v), last(x.g), last(x.beta), x.w_lam, x.b_lam, rule, c)
    assert normwise_error(od[:, :, None], o[:, :, 40:41]) < 1e-13
    assert normwise_error(cd.S, st.S) < 1e-13 and np.array_equal(cd.n, st.n)


def test_gla_closed_form_carry():
    """The closed-form GLA prefix carry equals the recurrence's final carry."""
    x = gla_inputs(2, 2, 70, 8, 121, "f32")
    _, st = _run(x)
    cf = gla_closed_form_carry(x.k, x.v, x.g)
    for a, b in ((cf.S, st.S), (cf.C, st.C), (cf.m, st.m)):
        assert normwise_error(a, b) < 1e-12
    assert np.array_equal(cf.n, st.n)


def test_carry_roundtrip_and_zero_carry():
    x = gla_inputs(1, 1, 5, 4, 131, "f32")
    o1, _ = _run(x)
    o2, _ = _run(x, carry=Carry.zeros(1, 1, 4, 4))
    assert np.array_equal(o1, o2)


def test_normwise_error_metric():
    y = np.zeros((2, 3, 4, 5))
    y[1, 2, 3, 4] = 2.0
    y[0, 0, 0, 0] = -4.0
    x = y.copy()
    x[1, 2, 0, 0] = 0.5
    assert normwise_error(x, y) == pytest.approx(0.25)
    assert normwise_error(y, y) == 0.0


# ---------------------------------------------------------------- generator / upload


def test_bf16_rounding_matches_torch():
    """The generator's bf16 values are bit-identical to what torch uploads (RNE)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, 1e-30, 3e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x), ref)
    r = bf16_round(x)
    assert np.array_equal(torch.from_numpy(r).to(torch.bfloat16).float().numpy(), r)


def test_generators_are_seeded_and_unit_keys():
    a = gla_inputs(1, 2, 16, 8, 5, "bf16")
    b = gla_inputs(1, 2, 16, 8, 5, "bf16")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.g, b.g)
    norms = np.linalg.norm(a.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(norms - 1) < 1e-2)
    f = gla_inputs(1, 2, 16, 8, 5, "f32")
    assert np.all(np.abs(np.linalg.norm(f.k.astype(np.float64), axis=-1) - 1) < 1e-6)
    gd = gdn_inputs(1, 2, 16, 8, 5, "f32")
    assert np.all((gd.beta > 0) & (gd.beta < 1)) and np.all(gd.g < 0)


def test_unit_keys_definition():
    """unit_keys: norm 1 along the last axis, direction kept, zero key stays zero, invariant to a
    positive rescale, idempotent -- pinned without re-typing the formula."""
    rng = np.random.default_rng(31)
    k = rng.standard_normal((2, 3, 5, 16)) * rng.uniform(0.1, 7.0, size=(2, 3, 5, 1))
    k[0, 1, 2] = 0.0
    u = unit_keys(k)
    n = np.linalg.norm(u, axis=-1)
    mask = np.ones_like(n, dtype=bool)
    mask[0, 1, 2] = False
    assert np.allclose(n[mask], 1.0, atol=1e-14)
    assert np.array_equal(u[0, 1, 2], np.zeros(16))
    cos = np.sum(u * k, axis=-1)[mask] / np.linalg.norm(k, axis=-1)[mask]
    assert np.allclose(cos, 1.0, atol=1e-14)  # same direction
    assert np.allclose(unit_keys(3.5 * k), u, atol=1e-15)
    assert np.allclose(unit_keys(u), u, atol=1e-15)
    # a hand case: (3, 4) -> (0.6, 0.8)
    assert np.allclose(unit_keys(np.array([3.0, 4.0])), [0.6, 0.8], atol=1e-15)


def test_pack_upper_layout():
    """pack_upper: a hand case, the position of every entry against the closed-form offset of a
    row-by-row upper triangle, the entry count, and the weighted-sum invariant (off-diagonal
    entries stand for two matrix entries)."""
    C3 = np.array([[1.0, 2.0, 3.0], [2.0, 4.0, 5.0], [3.0, 5.0, 6.0]])
    assert np.array_equal(pack_upper(C3), [1.0, 2.0, 3.0, 4.0, 5.0, 6.0])
    d = 7
    # entry (i, j), i <= j, tagged by a value that names it
    M = np.array([[100.0 * min(i, j) + max(i, j) for j in range(d)] for i in range(d)])
    p = pack_upper(M)
    assert p.shape == (d * (d + 1) // 2,)
    for i in range(d):
        for j in range(i, d):
            off = i * d - i * (i - 1) // 2 + (j - i)
            assert p[off] == 100.0 * i + j, (i, j, off)
    rng = np.random.default_rng(41)
    K = rng.standard_normal((2, 3, 20, 16))
    C = np.swapaxes(K, -1, -2) @ K
    pc = pack_upper(C)
    diag = np.array([1.0 if i == j else 2.0 for i in range(16) for j in range(i, 16)])
    assert np.allclose((pc * diag).sum(axis=-1), C.sum(axis=(-1, -2)), rtol=1e-13)


def test_unpack_upper_round_trip():
    """unpack_upper inverts pack_upper exactly on symmetric matrices (batched), returns a
    symmetric matrix for any packed vector, and rejects a wrong length."""
    rng = np.random.default_rng(42)
    K = rng.standard_normal((3, 2, 40, 12)).astype(np.float32)
    C = np.swapaxes(K, -1, -2) @ K
    C = (C + np.swapaxes(C, -1, -2)) / 2
    assert np.array_equal(unpack_upper(pack_upper(C), 12), C)
    p = rng.standard_normal(12 * 13 // 2)
    U = unpack_upper(p, 12)
    assert np.array_equal(U, U.T)
    assert np.array_equal(pack_upper(U), p)
    with pytest.raises(ValueError):
        unpack_upper(p[:-1], 12)

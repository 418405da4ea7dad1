"""Pins of the key-covariance subspace diagnostic in the oracle (``oracle/subspace.py``) against
things other than itself: numpy's covariance, diagonal and hand-solved 2 x 2 spectra, the
spectral reconstruction, closed-form alignments of keys inside / orthogonal to the subspace,
rotation and scale invariance, and a hand-computed Δμ.  A second part plants slips into a
private copy of the module and checks that the pins reject each one."""

import os
import types

import numpy as np
import pytest

from oracle import covariance_from_sums, delta_mu, subspace_alignment, top_eigen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "subspace.py")


def test_covariance_from_sums_is_numpy_cov():
    rng = np.random.default_rng(51)
    K = rng.standard_normal((2, 3, 40, 8))
    C = np.swapaxes(K, -1, -2) @ K
    m = K.sum(axis=-2)
    n = np.full((2, 3), 40)
    S = covariance_from_sums(C, m, n)
    for b in range(2):
        for h in range(3):
            assert np.allclose(S[b, h], np.cov(K[b, h].T, bias=True), atol=1e-13)
    assert np.array_equal(covariance_from_sums(C[:1, :1], m[:1, :1], np.zeros((1, 1))), np.zeros((1, 1, 8, 8)))


def test_top_eigen_diagonal_and_hand_case():
    w, U = top_eigen(np.diag([0.5, 3.0, 0.1, 2.0]), 2)
    assert np.allclose(w, [3.0, 2.0, 0.5, 0.1], atol=1e-15)
    assert np.allclose(U, [[0, 1, 0, 0], [0, 0, 0, 1]], atol=1e-15)  # axes, sign made positive
    w, U = top_eigen(np.array([[2.0, 1.0], [1.0, 2.0]]), 1)
    assert np.allclose(w, [3.0, 1.0], atol=1e-14)
    assert np.allclose(U, [[1 / np.sqrt(2), 1 / np.sqrt(2)]], atol=1e-14)
    w, U = top_eigen(np.array([[2.0, -1.0], [-1.0, 2.0]]), 2)
    assert np.allclose(w, [3.0, 1.0], atol=1e-14)
    # largest-magnitude entry positive; equal magnitudes: the lower index decides
    assert np.allclose(U, [[1 / np.sqrt(2), -1 / np.sqrt(2)], [1 / np.sqrt(2), 1 / np.sqrt(2)]], atol=1e-14)


def test_top_eigen_reconstructs_and_is_orthonormal():
    rng = np.random.default_rng(52)
    X = rng.standard_normal((3, 64, 12))
    S = np.swapaxes(X, -1, -2) @ X / 64
    w, U = top_eigen(S, 12)
    assert np.all(np.diff(w, axis=-1) <= 0)
    eye = np.broadcast_to(np.eye(12), (3, 12, 12))
    assert np.allclose(U @ np.swapaxes(U, -1, -2), eye, atol=1e-12)
    rec = np.swapaxes(U, -1, -2) @ (w[..., :, None] * U)
    assert np.allclose(rec, S, atol=1e-12)
    # each row is an eigenvector: S u = w u
    assert np.allclose(np.einsum("bij,bkj->bki", S, U), w[..., None] * U, atol=1e-12)


def test_alignment_closed_forms():
    d = 10
    U = np.eye(d)[[2, 5, 7]]                      # subspace of axes 2, 5, 7
    rng = np.random.default_rng(53)
    K = rng.standard_normal((6, d))
    a = subspace_alignment(K, U)
    ref = (K[:, 2] ** 2 + K[:, 5] ** 2 + K[:, 7] ** 2) / np.sum(K * K, axis=-1)
    assert np.allclose(a, ref, atol=1e-15)
    inside = np.zeros((2, d))
    inside[0, [2, 7]] = [1.0, -3.0]
    inside[1, 5] = 0.25
    assert np.allclose(subspace_alignment(inside, U), 1.0, atol=1e-15)
    outside = np.zeros((2, d))
    outside[0, [0, 9]] = [2.0, 1.0]
    assert np.array_equal(subspace_alignment(outside, U), [0.0, 0.0])  # second row is the zero key
    assert np.allclose(subspace_alignment(7.5 * K, U), a, atol=1e-15)


def test_alignment_rotation_invariant():
    rng = np.random.default_rng(54)
    d, r = 16, 4
    X = rng.standard_normal((80, d)) * np.linspace(3, 0.2, d)
    S = X.T @ X / 80
    K = rng.standard_normal((30, d))
    R, _ = np.linalg.qr(rng.standard_normal((d, d)))
    _, U = top_eigen(S, r)
    _, U2 = top_eigen(R @ S @ R.T, r)
    assert np.allclose(subspace_alignment(K @ R.T, U2), subspace_alignment(K, U), atol=1e-12)


def test_delta_mu_hand_case_and_sign():
    a = np.array([[0.9, 0.1, 0.2, 0.8]])
    needle = np.array([[False, True, False, False]])
    assert np.allclose(delta_mu(a, needle), [0.1 - (0.9 + 0.2 + 0.8) / 3], atol=1e-15)
    assert np.isnan(delta_mu(a, np.zeros_like(needle)))[0]
    # haystack keys spread over a 16-dim subspace, needle keys orthogonal to it: Δμ = -1
    rng = np.random.default_rng(55)
    d, T = 64, 400
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    hay = rng.standard_normal((T, 16)) @ basis[:, :16].T
    nd = rng.standard_normal((5, 8)) @ basis[:, 40:48].T
    K = np.concatenate([hay, nd])
    msk = np.r_[np.zeros(T, bool), np.ones(5, bool)]
    S = covariance_from_sums(K.T @ K, K.sum(0), len(K))
    _, U = top_eigen(S, 16)
    dm = delta_mu(subspace_alignment(K, U), msk)
    assert dm < 0 and np.isclose(dm, -1.0, atol=1e-3)


MUTATIONS = {
    "ascending_eigenvalues": ("    w = w[..., ::-1]\n    U = np.swapaxes(V[..., :, ::-1], -1, -2)[..., :r, :]",
                              "    U = np.swapaxes(V, -1, -2)[..., :r, :]"),
    "columns_as_rows": ("    U = np.swapaxes(V[..., :, ::-1], -1, -2)[..., :r, :]", "    U = V[..., ::-1, :][..., :r, :]"),
    "unnormalised_alignment": ("num / np.where(den > 0, den, 1.0)", "num"),
    "delta_sign": ("mn - md, np.nan", "md - mn, np.nan"),
    "mean_not_centred": ("S = C / safe[..., None, None] - mu[..., :, None] * mu[..., None, :]",
                         "S = C / safe[..., None, None]"),
}


def _mutant(name):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType(f"subspace_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _pins_hold(m) -> bool:
    try:
        rng = np.random.default_rng(56)
        K = rng.standard_normal((30, 6)) + 0.5
        S = m.covariance_from_sums(K.T @ K, K.sum(0), 30)
        if not np.allclose(S, np.cov(K.T, bias=True), atol=1e-12):
            return False
        w, U = m.top_eigen(np.diag([0.5, 3.0, 0.1, 2.0]), 2)
        if not (np.allclose(w, [3.0, 2.0, 0.5, 0.1]) and np.allclose(U, [[0, 1, 0, 0], [0, 0, 0, 1]])):
            return False
        w, U = m.top_eigen(np.array([[2.0, 1.0], [1.0, 3.0]]), 1)
        X = np.array([[2.0, 1.0], [1.0, 3.0]])
        if not np.allclose(X @ U[0], w[0] * U[0], atol=1e-12):
            return False
        Ua = np.eye(5)[[1, 3]]
        k = np.array([[1.0, 2.0, 0.0, 2.0, 0.0]])
        if not np.allclose(m.subspace_alignment(k, Ua), [8.0 / 9.0]):
            return False
        return bool(np.allclose(m.delta_mu(np.array([[0.9, 0.1, 0.2, 0.8]]), np.array([[0, 1, 0, 0]], bool)),
                                [0.1 - 1.9 / 3]))
    except Exception:
        return False


def test_unmutated_subspace_oracle_passes_pins():
    import oracle.subspace as real
    assert _pins_hold(real)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_subspace_mutation_is_caught(name):
    assert not _pins_hold(_mutant(name)), f"pins did not catch mutation {name}"

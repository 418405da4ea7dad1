"""Plain fp64 CPU reference of the key-covariance subspace diagnostic (test infrastructure
only; nothing in the product path imports it).

The 10100.com write-up of the CCQ paper, section "记忆体检", describes a geometric check of a
linear-attention memory: Δμ, the difference between how strongly the target (needle) keys and
the distractor keys align with the top-16 eigen-subspace of the key covariance; a negative
Δμ means the needle sits further from the high-variance subspace, which is the premise the
cleaned query relies on.  The page gives the idea, not a formula.  The reading taken here
(stated in the design notes): with U_r the top-r unit eigenvectors of Σ (the covariance the
method's statistics hold, gist.science summary §2 "理论推导"),

    a(k)  = |U_r^T k|^2 / |k|^2     (energy fraction of key k in the subspace; 0 for k = 0)
    Δμ    = mean of a over needle keys - mean of a over distractor keys.

Shapes: Sigma [..., d, d]; K [..., T, d]; needle mask [..., T] (bool).
"""

from __future__ import annotations

import numpy as np

f64 = np.float64

__all__ = ["covariance_from_sums", "top_eigen", "subspace_alignment", "delta_mu"]


def covariance_from_sums(C, m, n) -> np.ndarray:
    """Sigma = C / n - (m / n)(m / n)^T from the statistics kept as sums (C = sum k k^T,
    m = sum k, n tokens): Cbar - mu mu^T, gist.science summary §2 "理论推导".  n <= 0 gives 0."""
    C = np.asarray(C, dtype=f64)
    m = np.asarray(m, dtype=f64)
    n = np.asarray(n, dtype=f64)
    safe = np.where(n > 0, n, 1.0)
    mu = m / safe[..., None]
    S = C / safe[..., None, None] - mu[..., :, None] * mu[..., None, :]
    return np.where((n > 0)[..., None, None], S, 0.0)


def top_eigen(Sigma, r: int):
    """Eigenvalues of the symmetric Sigma in descending order ([..., d]) and the top-r unit
    eigenvectors as rows ([..., r, d]), each with its largest-magnitude entry positive (the
    lowest index among equal magnitudes).  LAPACK's symmetric eigensolver (numpy.linalg.eigh)
    is the step that finds them."""
    S = np.asarray(Sigma, dtype=f64)
    w, V = np.linalg.eigh(S)                    # ascending, eigenvectors as columns
    w = w[..., ::-1]
    U = np.swapaxes(V[..., :, ::-1], -1, -2)[..., :r, :]
    idx = np.argmax(np.abs(U), axis=-1)         # first index of the largest magnitude
    sign = np.sign(np.take_along_axis(U, idx[..., None], axis=-1))
    sign = np.where(sign == 0, 1.0, sign)
    return w, U * sign


def subspace_alignment(K, U) -> np.ndarray:
    """a_t = |U K_t|^2 / |K_t|^2 for every row K_t of K [..., T, d], with U [..., r, d] holding
    orthonormal rows; 0 where K_t = 0."""
    K = np.asarray(K, dtype=f64)
    U = np.asarray(U, dtype=f64)
    y = K @ np.swapaxes(U, -1, -2)              # [..., T, r]
    num = np.sum(y * y, axis=-1)
    den = np.sum(K * K, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def delta_mu(align, needle) -> np.ndarray:
    """mean(a over needle tokens) - mean(a over the other tokens), per leading index; NaN
    where either set is empty."""
    a = np.asarray(align, dtype=f64)
    msk = np.asarray(needle, dtype=bool)
    nn = msk.sum(axis=-1)
    nd = (~msk).sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        mn = np.where(msk, a, 0.0).sum(axis=-1) / nn
        md = np.where(~msk, a, 0.0).sum(axis=-1) / nd
    return np.where((nn > 0) & (nd > 0), mn - md, np.nan)

"""Plain fp64 CPU reference of the CCQ read step (test infrastructure only).

Two forms are kept, both in float64 NumPy:

* ``ccq_recurrent`` is the plain per-token definition.  It is THE oracle the
  HIP path is compared against.
* ``ccq_chunked`` is the same result reached by unrolling the recurrence inside
  chunks of L tokens (the statistics may follow the backbone's own recurrent or
  chunked form, gist.science summary §2 "机制").  It exists to pin that algebra
  against the plain definition.

Notation follows the pages: keys k_t (unit norm), queries q_t, values v_t; the
running undecayed statistics are the key sum m, the second-moment sum C and the
count n, so mu_t = m/n and Cbar_t = C/n; Sigma_t = Cbar_t - mu_t mu_t^T.
Shapes: q, k [B, H, T, d_k]; v [B, H, T, d_v]; state S [B, H, d_v, d_k].
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Carry",
    "sigmoid",
    "key_covariance",
    "unit_keys",
    "ccq_recurrent",
    "ccq_chunked",
    "ccq_decode_step",
    "gla_closed_form_carry",
    "normwise_error",
    "pack_upper",
    "unpack_upper",
]

f64 = np.float64


@dataclasses.dataclass
class Carry:
    """The recurrent state of one layer: the write-rule state S plus the key
    statistics (one d_k x d_k matrix and one d_k vector per head, gist.science
    summary §2 "机制"), stored as sums with an explicit token count."""

    S: np.ndarray  # [B, H, d_v, d_k]
    C: np.ndarray  # [B, H, d_k, d_k]  sum_j k_j k_j^T
    m: np.ndarray  # [B, H, d_k]       sum_j k_j
    n: np.ndarray  # [B, H] int64      number of tokens seen

    @staticmethod
    def zeros(B: int, H: int, d_k: int, d_v: int) -> "Carry":
        return Carry(np.zeros((B, H, d_v, d_k), f64), np.zeros((B, H, d_k, d_k), f64),
                     np.zeros((B, H, d_k), f64), np.zeros((B, H), np.int64))

    def copy(self) -> "Carry":
        return Carry(self.S.astype(f64, copy=True), self.C.astype(f64, copy=True),
                     self.m.astype(f64, copy=True), np.array(self.n, dtype=np.int64, copy=True))


def sigmoid(x):
    """Logistic function; sigmoid(-inf) = 0 exactly (the gate's sigma in the
    gist.science summary §2 "机制")."""
    x = np.asarray(x, dtype=f64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def key_covariance(K: np.ndarray) -> np.ndarray:
    """Sigma_t of the keys K[:t] ([t, d]): Cbar_t - mu_t mu_t^T with the running
    mean and second moment over j <= t (gist.science summary §2 "理论推导",
    second-order expansion of the log-partition)."""
    K = np.asarray(K, dtype=f64)
    t = K.shape[0]
    mu = K.sum(axis=0) / t
    Cbar = K.T @ K / t
    return Cbar - np.outer(mu, mu)


def unit_keys(k, eps: float = 1e-12) -> np.ndarray:
    """Keys scaled to unit L2 norm along the last axis, k / max(|k|, eps), in fp64.

    Unit keys are the precondition of the method's eigenvalue bound (10100.com write-up,
    section "方法解析"); when a caller asks the library to normalise, this is the definition
    it is held to (the eps floor, which keeps an all-zero key at zero, is this library's
    reading: the pages are silent on it)."""
    k = np.asarray(k, dtype=f64)
    nrm = np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    return k / np.maximum(nrm, eps)


def _as64(x):
    return None if x is None else np.asarray(x, dtype=f64)


def _check_rule(rule: str, g, beta, k):
    if rule == "gla":
        if g.shape != k.shape:
            raise ValueError("GLA takes log alpha per key channel: g must match k's shape")
    elif rule == "gdn":
        if g.shape != k.shape[:-1] or beta is None or beta.shape != k.shape[:-1]:
            raise ValueError("Gated DeltaNet takes scalar log alpha and beta per token")
    else:
        raise ValueError(f"unknown write rule {rule!r}")


def ccq_recurrent(q, k, v, g, beta, w_lam, b_lam, rule: str, carry: Optional[Carry] = None,
                  record: bool = False, record_sigma: bool = False):
    """Per-token CCQ read on a GLA or Gated DeltaNet backbone, in fp64.

    For each (b, h) and t = 1..T, in this order:
      1. n += 1; C += k_t k_t^T; m += k_t  -- statistics include token t and are
         never decayed (summary §2 "理论推导" sums over j <= t; write-up section
         "代价与边界" calls the covariance undecayed).
      2. Sigma_t = C/n - (m/n)(m/n)^T  (summary §2 "理论推导").
      3. lambda_t = sigmoid(W_lambda q_t + b_lambda), one scalar per token and
         head (summary §2 "机制"; write-up section "方法解析", point 1).
      4. q_clean = q_t - lambda_t Sigma_t q_t  (summary §2 "机制").
      5. Write, unchanged (summary §2 "集成"):
         GLA  S_t = S_{t-1} diag(alpha_t) + v_t k_t^T, alpha_t = exp(g_t) per key channel;
         GDN  S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, alpha_t = exp(g_t).
      6. o_t = S_t q_clean, with S_t the state after token t's write (§2 "集成").

    Returns (o [B,H,T,d_v], final Carry[, record]) where record holds lambda
    [B,H,T], q_clean [B,H,T,d_k] and, if asked, Sigma_t [B,H,T,d_k,d_k].
    """
    q, k, v, g, beta = (_as64(x) for x in (q, k, v, g, beta))
    w_lam = np.asarray(w_lam, dtype=f64)
    b_lam = np.asarray(b_lam, dtype=f64)
    _check_rule(rule, g, beta, k)
    B, H, T, d_k = q.shape
    d_v = v.shape[-1]
    st = Carry.zeros(B, H, d_k, d_v) if carry is None else carry.copy()
    o = np.zeros((B, H, T, d_v), f64)
    lam_rec = np.zeros((B, H, T), f64)
    qc_rec = np.zeros((B, H, T, d_k), f64)
    sig_rec = np.zeros((B, H, T, d_k, d_k), f64) if record_sigma else None
    for t in range(T):
        qt, kt, vt = q[:, :, t], k[:, :, t], v[:, :, t]
        # 1. undecayed statistics, token t included
        st.n = st.n + 1
        st.C = st.C + kt[..., :, None] * kt[..., None, :]
        st.m = st.m + kt
        # 2. covariance from the running mean and second moment
        nn = st.n.astype(f64)
        mu = st.m / nn[..., None]
        Cbar = st.C / nn[..., None, None]
        Sigma = Cbar - mu[..., :, None] * mu[..., None, :]
        # 3. gate
        lam = sigmoid(np.einsum("bhd,hd->bh", qt, w_lam) + b_lam[None, :])
        # 4. cleaned query
        q_clean = qt - lam[..., None] * np.matmul(Sigma, qt[..., None])[..., 0]
        # 5. write rule
        if rule == "gla":
            st.S = st.S * np.exp(g[:, :, t])[..., None, :] + vt[..., :, None] * kt[..., None, :]
        else:
            a = np.exp(g[:, :, t])[..., None, None]
            bt = beta[:, :, t][..., None, None]
            Sk = np.matmul(st.S, kt[..., None])  # [B,H,d_v,1]
            st.S = a * (st.S - bt * Sk * kt[..., None, :]) + bt * vt[..., :, None] * kt[..., None, :]
        # 6. read with the cleaned query
        o[:, :, t] = np.matmul(st.S, q_clean[..., None])[..., 0]
        if record:
            lam_rec[:, :, t] = lam
            qc_rec[:, :, t] = q_clean
            if record_sigma:
                sig_rec[:, :, t] = Sigma
    if record:
        rec = dict(lam=lam_rec, q_clean=qc_rec)
        if record_sigma:
            rec["sigma"] = sig_rec
        return o, st, rec
    return o, st


def _tril(n: int, strict: bool = False) -> np.ndarray:
    return np.tril(np.ones((n, n), dtype=bool), k=-1 if strict else 0)


def ccq_chunked(q, k, v, g, beta, w_lam, b_lam, rule: str, carry: Optional[Carry] = None,
                chunk: int = 64):
    """The recurrence above, evaluated chunk by chunk (fp64 algebra check).

    Inside a chunk of rows i = 1..L with carry (S0, C0, m0, n0):
      CCQ: s_i = m0 + sum_{j<=i} k_j, n_i = n0 + i,
           R = Q C0 + tril_incl(Q K^T) K   (row i is C_i q_i),
           u_i = R_i / n_i - s_i (s_i . q_i) / n_i^2  (row i is Sigma_i q_i),
           q_clean_i = q_i - lambda_i u_i.
      GLA: with Bc_i = sum_{j<=i} g_j (per channel),
           O = (Qc * e^Bc) S0^T + tril_incl(A) V,  A_ij = sum_c qc_ic k_jc e^{Bc_ic - Bc_jc},
           S_L = S0 diag(e^{Bc_L}) + V^T (K * e^{Bc_L - Bc}).
      GDN: with gamma_i = prod_{j<=i} alpha_j and Gam_ij = gamma_i / gamma_j,
           delta_i = beta_i (v_i - alpha_i S_{i-1} k_i) solves
           (I + A) Delta = diag(beta) (V - diag(gamma) K S0^T),  A_ij = beta_i Gam_ij k_i.k_j (j < i);
           Tm = (I + A)^{-1}, U = Tm diag(beta) V, W = Tm diag(beta gamma) K, Delta = U - W S0^T,
           O = diag(gamma) Qc S0^T + (tril_incl(Qc K^T) * Gam) Delta,
           S_L = gamma_L S0 + Delta^T diag(gamma_L / gamma) K.
      carry: C0 += K^T K, m0 += sum K, n0 += L.
    """
    q, k, v, g, beta = (_as64(x) for x in (q, k, v, g, beta))
    w_lam = np.asarray(w_lam, dtype=f64)
    b_lam = np.asarray(b_lam, dtype=f64)
    _check_rule(rule, g, beta, k)
    B, H, T, d_k = q.shape
    d_v = v.shape[-1]
    st = Carry.zeros(B, H, d_k, d_v) if carry is None else carry.copy()
    o = np.zeros((B, H, T, d_v), f64)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        L = t1 - t0
        Q, K, V = q[:, :, t0:t1], k[:, :, t0:t1], v[:, :, t0:t1]
        incl = _tril(L)
        # --- CCQ statistics and cleaned query
        s = st.m[..., None, :] + np.cumsum(K, axis=-2)
        n_i = st.n[..., None].astype(f64) + np.arange(1, L + 1, dtype=f64)
        Pm = np.where(incl, Q @ np.swapaxes(K, -1, -2), 0.0)
        R = Q @ np.swapaxes(st.C, -1, -2) + Pm @ K
        sq = np.sum(s * Q, axis=-1)
        u = R / n_i[..., None] - s * (sq / n_i ** 2)[..., None]
        lam = sigmoid(np.einsum("bhld,hd->bhl", Q, w_lam) + b_lam[None, :, None])
        Qc = Q - lam[..., None] * u
        S0T = np.swapaxes(st.S, -1, -2)  # [B,H,d_k,d_v]
        if rule == "gla":
            G = g[:, :, t0:t1]
            Bc = np.cumsum(G, axis=-2)  # [B,H,L,d_k]
            inter = (Qc * np.exp(Bc)) @ S0T
            diff = Bc[..., :, None, :] - Bc[..., None, :, :]  # [B,H,L(i),L(j),d_k]
            diff = np.where(incl[..., None], diff, -np.inf)
            A = np.einsum("bhic,bhjc,bhijc->bhij", Qc, K, np.exp(diff))
            o[:, :, t0:t1] = inter + A @ V
            BL = Bc[..., -1, :]
            st.S = st.S * np.exp(BL)[..., None, :] + np.swapaxes(V, -1, -2) @ (K * np.exp(BL[..., None, :] - Bc))
        else:
            lg = np.cumsum(g[:, :, t0:t1], axis=-1)  # log gamma, [B,H,L]
            bt = beta[:, :, t0:t1]
            gam = np.exp(lg)
            ldiff = lg[..., :, None] - lg[..., None, :]
            Gam = np.where(incl, np.exp(np.where(incl, ldiff, 0.0)), 0.0)
            KK = K @ np.swapaxes(K, -1, -2)
            A = np.where(_tril(L, strict=True), bt[..., :, None] * Gam * KK, 0.0)
            Tm = np.linalg.inv(np.eye(L) + A)
            U = Tm @ (bt[..., None] * V)
            W = Tm @ ((bt * gam)[..., None] * K)
            Delta = U - W @ S0T
            QK = np.where(incl, Qc @ np.swapaxes(K, -1, -2), 0.0)
            o[:, :, t0:t1] = gam[..., None] * (Qc @ S0T) + (QK * Gam) @ Delta
            gL = gam[..., -1]
            st.S = gL[..., None, None] * st.S + np.swapaxes(Delta, -1, -2) @ ((gL[..., None] / gam)[..., None] * K)
        st.C = st.C + np.swapaxes(K, -1, -2) @ K
        st.m = st.m + K.sum(axis=-2)
        st.n = st.n + L
    return o, st


def ccq_decode_step(q, k, v, g, beta, w_lam, b_lam, rule: str, carry: Carry):
    """One decode step: the recurrence with a single new token per (seq, head).

    q, k [N, H, d_k]; v [N, H, d_v]; g GLA [N, H, d_k] / GDN [N, H]; beta GDN [N, H].
    Returns (o [N, H, d_v], updated Carry)."""
    ex = lambda x: None if x is None else np.asarray(x, dtype=f64)[:, :, None]  # noqa: E731
    o, st = ccq_recurrent(ex(q), ex(k), ex(v), ex(g), ex(beta), w_lam, b_lam, rule, carry)
    return o[:, :, 0], st


def gla_closed_form_carry(k, v, g) -> Carry:
    """Carry after a GLA prefix, written in closed form rather than by recurrence:
    S = sum_j v_j (k_j * exp(sum_{j' > j} g_j'))^T, C = sum_j k_j k_j^T,
    m = sum_j k_j, n = T.  k, v, g are [B, H, T, d]."""
    k, v, g = (np.asarray(x, dtype=f64) for x in (k, v, g))
    T = k.shape[-2]
    after = np.cumsum(g[..., ::-1, :], axis=-2)[..., ::-1, :] - g  # sum over j' > j
    S = np.swapaxes(v, -1, -2) @ (k * np.exp(after))
    C = np.swapaxes(k, -1, -2) @ k
    m = k.sum(axis=-2)
    n = np.full(k.shape[:2], T, dtype=np.int64)
    return Carry(S, C, m, n)


def pack_upper(C) -> np.ndarray:
    """Packed form of a symmetric [..., d, d] statistic: its upper triangle, row by row
    (C[0][0..d-1], C[1][1..d-1], ..., C[d-1][d-1]), d (d + 1) / 2 entries.

    The second-moment sum is the one state of the method that is symmetric (a sum of k k^T,
    gist.science summary §2 "理论推导"); keeping one triangle is the compact statistic state
    the 10100.com write-up's section "代价与边界" motivates by the memory the extra
    d_k x d_k matrix costs at inference.  The row order is this library's reading: the pages
    fix no layout."""
    C = np.asarray(C)
    d = C.shape[-1]
    if C.shape[-2] != d:
        raise ValueError("pack_upper takes square matrices")
    iu, ju = np.triu_indices(d)
    return C[..., iu, ju]


def unpack_upper(p, d: int) -> np.ndarray:
    """Inverse of ``pack_upper``: the symmetric [..., d, d] matrix whose upper triangle,
    row by row, is p[..., :d (d + 1) / 2]."""
    p = np.asarray(p)
    if p.shape[-1] != d * (d + 1) // 2:
        raise ValueError(f"a packed {d}x{d} triangle has {d * (d + 1) // 2} entries, got {p.shape[-1]}")
    out = np.zeros(p.shape[:-1] + (d, d), dtype=p.dtype)
    iu, ju = np.triu_indices(d)
    out[..., iu, ju] = p
    out[..., ju, iu] = p
    return out


def normwise_error(x, y) -> float:
    """max over (b, h) slabs of max|x - y| / max|y| (arrays [B, H, ...])."""
    x = np.asarray(x, dtype=f64)
    y = np.asarray(y, dtype=f64)
    if x.shape != y.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {y.shape}")
    if x.size == 0:
        return 0.0
    lead = x.shape[:2] if x.ndim >= 3 else x.shape[:1]
    xs = x.reshape(int(np.prod(lead)), -1)
    ys = y.reshape(int(np.prod(lead)), -1)
    num = np.max(np.abs(xs - ys), axis=1)
    den = np.max(np.abs(ys), axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))

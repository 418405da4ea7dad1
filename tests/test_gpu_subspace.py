"""Key-covariance subspace diagnostic: HIP kernels through the C ABI vs the fp64 oracle.

Tolerances, derived from the fp32 method (the Householder reduction is backward stable to a few
d * 2^-24 of the matrix norm, bisection adds a few ulps, so the eigenvalues carry an absolute
error of order d * 2^-24 * lambda_max and an eigenvector one of that over the gap to its
neighbours; Gram-Schmidt twice keeps the basis orthonormal to a few ulps): eigenvalues within 2e-5 of
lambda_max; the rows of the basis within 2e-3 (the closest pair of the 16 leading eigenvalues of
these keys is about 1e-2 of lambda_max apart); per-key alignment and Δμ within 1e-4 (they depend
on the subspace only, whose gap to the rest of the spectrum is about 0.25 lambda_max).  The keys
come from ``subspace_keys`` (16 well-separated leading directions, needles every 64 tokens)."""

import numpy as np
import pytest

from curvature_conditioned_query_amd.inputs import subspace_keys, workload_inputs
from oracle import covariance_from_sums, delta_mu, pack_upper, subspace_alignment, top_eigen

from gpu_util import down, up

pytestmark = pytest.mark.gpu

EIG_TOL, BASIS_TOL, ALIGN_TOL = 2e-5, 2e-3, 1e-4


def _stats(k):
    """fp32 statistics of the keys (as a carry holds them), computed on the host."""
    K = k.astype(np.float64)
    C = (np.swapaxes(K, -1, -2) @ K).astype(np.float32)
    C = ((C + np.swapaxes(C, -1, -2)) / 2).astype(np.float32)
    m = K.sum(axis=-2).astype(np.float32)
    n = np.full(k.shape[:2], k.shape[2], dtype=np.int64)
    return C, m, n


def _oracle(C, m, n, k, r, needle):
    S = covariance_from_sums(C.astype(np.float64), m.astype(np.float64), n)
    w, U = top_eigen(S, r)
    a = subspace_alignment(k, U)
    return w, U, a, (None if needle is None else delta_mu(a, needle))


def _gpu(C, m, n, k, r, needle, dtype, packed=False):
    import torch
    from curvature_conditioned_query_amd import ccq_key_subspace
    Cd = torch.from_numpy(np.ascontiguousarray(pack_upper(C) if packed else C)).cuda()
    out = ccq_key_subspace(Cd, torch.from_numpy(m).cuda(), torch.from_numpy(n).cuda(), up(k, dtype), r=r,
                           needle=None if needle is None else torch.from_numpy(needle).cuda(), packed_cov=packed)
    torch.cuda.synchronize()
    return tuple(None if t is None else down(t) for t in out)


def _check(got, ref, tag, basis_tol=BASIS_TOL):
    w, U, a, dm = got
    wr, Ur, ar, dmr = ref
    lam = np.max(np.abs(wr), axis=-1, keepdims=True)
    ew = np.max(np.abs(w - wr) / lam)
    eU = np.max(np.abs(U - Ur))
    ea = np.max(np.abs(a - ar))
    msg = f"{tag}: eig err {ew:.2e} basis err {eU:.2e} align err {ea:.2e}"
    if dm is not None:
        msg += f" delta-mu {float(dm.ravel()[0]):+.4f} err {np.max(np.abs(dm - dmr)):.2e}"
    print(msg, flush=True)
    assert ew <= EIG_TOL, msg
    assert eU <= basis_tol, msg
    assert ea <= ALIGN_TOL, msg
    if dm is not None:
        assert np.max(np.abs(dm - dmr)) <= ALIGN_TOL, msg
        assert np.all(dm < 0), msg  # needles sit off the leading subspace of these keys


@pytest.mark.parametrize("d,dtype,packed", [(64, "f32", False), (128, "bf16", False), (128, "bf16", True),
                                            (64, "bf16", True)])
def test_subspace_matches_oracle(d, dtype, packed):
    k, needle = subspace_keys(2, 2, 700, d, 300 + d, dtype)
    C, m, n = _stats(k)
    got = _gpu(C, m, n, k, 16, needle, dtype, packed)
    _check(got, _oracle(C, m, n, k, 16, needle), f"d={d} {dtype} packed={packed}")


@pytest.mark.parametrize("r", [1, 5, 32])
def test_subspace_ranks(r):
    """Other subspace sizes; for r = 32 the cut falls inside the noise spectrum, so only what is
    unique there is compared: eigenvalues, and alignment / basis for r <= 16."""
    k, needle = subspace_keys(1, 2, 500, 128, 310 + r, "bf16", rank=max(r, 1) if r <= 16 else 16)
    C, m, n = _stats(k)
    w, U, a, _ = _gpu(C, m, n, k, r, None, "bf16")
    wr, Ur, ar, _ = _oracle(C, m, n, k, r, None)
    lam = np.max(np.abs(wr), axis=-1, keepdims=True)
    assert np.max(np.abs(w - wr) / lam) <= EIG_TOL
    assert U.shape == (1, 2, r, 128) and a.shape == (1, 2, 500)
    G = U @ np.swapaxes(U, -1, -2)
    assert np.allclose(G, np.broadcast_to(np.eye(r), G.shape), atol=1e-5)  # orthonormal rows
    assert np.all((a >= -1e-6) & (a <= 1 + 1e-5))
    if r <= 16:
        assert np.max(np.abs(U - Ur)) <= BASIS_TOL
        assert np.max(np.abs(a - ar)) <= ALIGN_TOL


def test_subspace_edge_cases():
    """A zero key aligns 0; an empty needle set gives NaN; a head with n = 0 has Sigma = 0
    (all eigenvalues 0, basis still orthonormal) while its neighbour is unaffected; T not a
    multiple of the 64-token block."""
    k, needle = subspace_keys(1, 2, 131, 64, 320, "f32")
    k[0, 0, 5] = 0.0
    C, m, n = _stats(k)
    n[0, 1] = 0
    needle[0, 1] = False
    w, U, a, dm = _gpu(C, m, n, k, 8, needle, "f32")
    assert a[0, 0, 5] == 0.0
    assert np.isnan(dm[0, 1]) and np.isfinite(dm[0, 0])
    assert np.array_equal(w[0, 1], np.zeros(64))
    G = U[0, 1] @ U[0, 1].T
    assert np.allclose(G, np.eye(8), atol=1e-6)
    ref = _oracle(C[:, :1], m[:, :1], n[:, :1], k[:, :1], 8, needle[:, :1])
    _check((w[:, :1], U[:, :1], a[:, :1], dm[:, :1]), ref, "edge head 0")


@pytest.mark.parametrize("T,r", [(40, 32), (10, 32)])
def test_subspace_rank_deficient(T, r):
    """Fewer keys than channels (Sigma has rank <= T - 1, so d - T + 1 eigenvalues are zero): the
    eigenvalues match; the basis rows are orthonormal; for T = 10 the top 32 reach into the zero
    cluster, where any orthonormal completion is correct, so the rows that are unique (the
    leading ones, r <= 8 here) are compared, and the alignment stays in [0, 1]."""
    k, _ = subspace_keys(1, 2, T, 128, 360 + T, "f32", rank=4)
    C, m, n = _stats(k)
    w, U, a, _ = _gpu(C, m, n, k, r, None, "f32")
    wr, Ur, _, _ = _oracle(C, m, n, k, r, None)
    lam = np.max(np.abs(wr), axis=-1, keepdims=True)
    ew = np.max(np.abs(w - wr) / lam)
    G = U @ np.swapaxes(U, -1, -2)
    eo = np.max(np.abs(G - np.eye(r)))
    print(f"rank-deficient T={T} r={r}: eig err {ew:.2e} orthonormality {eo:.2e}", flush=True)
    assert ew <= EIG_TOL
    assert eo <= 1e-5
    assert np.all((a >= -1e-6) & (a <= 1 + 1e-5))
    lead = 4  # the keys' four leading directions are well separated from the rest
    assert np.max(np.abs(U[..., :lead, :] - Ur[..., :lead, :])) <= BASIS_TOL


def test_subspace_repeated_eigenvalues():
    """Sigma = diag(values) with exact repeats (5 x3, 3 x2, then distinct values and a zero block):
    the eigenvalues are exact to rounding, the basis rows are orthonormal, and each group of equal
    eigenvalues is spanned correctly: the projector onto the top 3 (and top 5) rows equals the
    coordinate projector of those channels."""
    import torch
    from curvature_conditioned_query_amd import ccq_key_subspace
    d, r = 64, 8
    vals = np.zeros(d)
    vals[[7, 20, 41]] = 5.0
    vals[[3, 60]] = 3.0
    vals[[11, 12, 13]] = [2.0, 1.5, 1.0]
    vals[30:40] = 0.25
    n = np.array([[1000]], dtype=np.int64)
    C = (np.diag(vals) * 1000).astype(np.float32)[None, None]
    m = np.zeros((1, 1, d), np.float32)
    k = np.random.default_rng(370).standard_normal((1, 1, 70, d)).astype(np.float32)
    out = ccq_key_subspace(torch.from_numpy(C).cuda(), torch.from_numpy(m).cuda(), torch.from_numpy(n).cuda(),
                           torch.from_numpy(k).cuda(), r=r)
    torch.cuda.synchronize()
    w, U = down(out[0])[0, 0], down(out[1])[0, 0]
    ref = np.sort(vals)[::-1]
    assert np.max(np.abs(w - ref)) <= EIG_TOL * 5.0
    assert np.max(np.abs(U @ U.T - np.eye(r))) <= 1e-5
    for top, chans in ((3, [7, 20, 41]), (5, [7, 20, 41, 3, 60])):
        P = U[:top].T @ U[:top]
        Pr = np.zeros((d, d))
        Pr[chans, chans] = 1.0
        e = np.max(np.abs(P - Pr))
        print(f"repeated eigenvalues: projector onto the top {top} off by {e:.2e}", flush=True)
        assert e <= 1e-4
    for j, ch in zip(range(5, 8), (11, 12, 13)):  # distinct values: the unit vector itself
        assert np.max(np.abs(U[j] - np.eye(d)[ch])) <= 1e-5


def test_subspace_from_prefill_carry():
    """The statistics as ccq_fwd_chunked carries them (C, ksum, n after a GLA prefill of the
    keys), full and packed, feed the diagnostic; the oracle reads the same carry values."""
    import torch
    from curvature_conditioned_query_amd import ccq_fwd_chunked
    x = workload_inputs(0)
    kk, needle = subspace_keys(1, 2, 256, 64, 330, "f32")
    x.k = kk
    B, H, T, d, _ = x.shape
    dev = {nm: up(getattr(x, nm), "f32") for nm in ("q", "k", "v", "g")}
    w_l, b_l = torch.from_numpy(x.w_lam).cuda(), torch.from_numpy(x.b_lam).cuda()
    for packed in (False, True):
        S = torch.empty((B, H, d, d), device="cuda")
        C = torch.empty((B, H, d * (d + 1) // 2) if packed else (B, H, d, d), device="cuda")
        m = torch.empty((B, H, d), device="cuda")
        n = torch.empty((B, H), dtype=torch.int64, device="cuda")
        ccq_fwd_chunked("gla", dev["q"], dev["k"], dev["v"], dev["g"], None, w_l, b_l, carry_out=(S, C, m, n),
                        packed_cov=packed)
        from curvature_conditioned_query_amd import ccq_key_subspace
        out = ccq_key_subspace(C, m, n, dev["k"], r=16, needle=torch.from_numpy(needle).cuda(), packed_cov=packed)
        torch.cuda.synchronize()
        got = tuple(down(t) for t in out)
        Ch = down(C)
        if packed:
            from oracle import unpack_upper
            Ch = unpack_upper(Ch, d)
        _check(got, _oracle(Ch, down(m), down(n), kk, 16, needle), f"from carry packed={packed}")


def test_subspace_full_size_sampled():
    """The benchmark's shape (B=4, H=16, T=4096, d=128 bf16 keys, r = 16): every head on the GPU,
    sampled heads against the oracle."""
    k, needle = subspace_keys(4, 16, 4096, 128, 340, "bf16")
    C, m, n = _stats(k)
    got = _gpu(C, m, n, k, 16, needle, "bf16")
    for (b, h) in [(0, 0), (3, 15), (2, 7)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = _oracle(C[sl], m[sl], n[sl], k[sl], 16, needle[sl])
        _check(tuple(t[sl] for t in got), ref, f"full size head ({b},{h})")


@pytest.mark.parametrize("d", [64, 128])
def test_subspace_iteration_counts(d):
    """The optional bisection work per head: a zero statistic (n = 0) needs none; a full
    covariance needs about log_{G+1}(2^23) rounds per eigenvalue with G = 512 / d points per
    round (8 at d = 64, 10 at d = 128), far below the cap of 40."""
    import torch
    from curvature_conditioned_query_amd import ccq_key_subspace
    k, _ = subspace_keys(1, 2, 300, d, 350, "bf16")
    C, m, n = _stats(k)
    n[0, 0] = 0
    it = torch.full((1, 2), -1, dtype=torch.int32, device="cuda")
    ccq_key_subspace(torch.from_numpy(C).cuda(), torch.from_numpy(m).cuda(), torch.from_numpy(n).cuda(),
                     up(k, "bf16"), r=16, iters=it)
    torch.cuda.synchronize()
    s = it.cpu().numpy()
    print(f"d={d} multisection rounds per head {s}", flush=True)
    assert s[0, 0] == 0
    assert 6 * d <= s[0, 1] <= 14 * d

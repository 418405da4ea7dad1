"""Decode-step parity: HIP kernel through the C ABI vs the fp64 oracle."""

import numpy as np
import pytest

from curvature_conditioned_query_amd.inputs import decode_tokens, gdn_inputs, gla_inputs, structured_inputs
from oracle import Carry, ccq_decode_step, ccq_recurrent, normwise_error, pack_upper, unit_keys

from gpu_util import down, up, up_carry

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
# The state is fp32 in both storage modes and the step is a handful of fp32 ops per element.
STATE_TOL = 1e-5


def _prefix_carry(rule, N, H, d, T, seed):
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(N, H, T, d, seed, "f32")
    _, c = ccq_recurrent(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule)
    return c


def _run_steps(gpu_lib, rule, dtype, N, H, d, steps, seed, structured=False, packed_cov=False,
               normalize_keys=False):
    import torch
    from curvature_conditioned_query_amd import ccq_decode_step as gpu_step
    carry = _prefix_carry(rule, N, H, d, 37, seed)
    (S, C, m, n), (S64, C64, m64, n64) = up_carry(carry)
    if packed_cov:
        C = torch.from_numpy(np.ascontiguousarray(pack_upper(C64.astype(np.float32)))).cuda()
    ref = Carry(S64, C64, m64, n64)
    for s in range(steps):
        tok = decode_tokens(rule, N, H, d, seed + 1 + s, dtype)
        if structured:
            sx = structured_inputs(rule, N, H, 1, d, seed + 100 + s, dtype)
            tok.update(k=sx.k[:, :, 0], w_lam=sx.w_lam, b_lam=sx.b_lam)
        k_in = tok["k"]
        if normalize_keys:  # a raw key of any scale; the oracle gets the unit key
            k_in = (tok["k"] * np.random.default_rng(seed + 50 + s).uniform(0.05, 20.0, size=(N, H, 1)))
            k_in = k_in.astype(np.float32)
            if dtype == "bf16":
                from curvature_conditioned_query_amd.inputs import bf16_round
                k_in = bf16_round(k_in)
        o = gpu_step(rule, up(tok["q"], dtype), up(k_in, dtype), up(tok["v"], dtype), up(tok["g"], dtype),
                     up(tok["beta"], dtype), torch.from_numpy(tok["w_lam"]).cuda(),
                     torch.from_numpy(tok["b_lam"]).cuda(), S, C, m, n, packed_cov=packed_cov,
                     normalize_keys=normalize_keys)
        torch.cuda.synchronize()
        k_ref = unit_keys(k_in) if normalize_keys else tok["k"]
        o_ref, ref = ccq_decode_step(tok["q"], k_ref, tok["v"], tok["g"], tok["beta"], tok["w_lam"],
                                     tok["b_lam"], rule, ref)
        err = normwise_error(down(o), o_ref)
        print(f"decode {rule} {dtype} d={d} packed={packed_cov} step {s}: o err {err:.3e}", flush=True)
        assert err <= TOL[dtype]
        # a bf16 key normalised in fp32 on the GPU vs fp64 in the oracle
        state_tol = 1e-4 if (normalize_keys and dtype == "bf16") else STATE_TOL
        assert normwise_error(down(S), ref.S) <= state_tol
        C_ref = pack_upper(ref.C) if packed_cov else ref.C
        assert normwise_error(down(C), C_ref) <= state_tol
        assert normwise_error(down(m)[:, :, :, None], ref.m[:, :, :, None]) <= STATE_TOL
        assert np.array_equal(down(n), ref.n)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_matches_oracle(gpu_lib, rule, dtype, d):
    _run_steps(gpu_lib, rule, dtype, N=3, H=2, d=d, steps=3, seed=500 + d)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_packed_cov(gpu_lib, rule, dtype, d):
    """C as the packed upper triangle (the packed-statistics flag): o, S and the packed C after
    three steps match the oracle, whose C is packed for the comparison."""
    _run_steps(gpu_lib, rule, dtype, N=3, H=2, d=d, steps=3, seed=520 + d, packed_cov=True)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_decode_packed_cov_normalize_keys(gpu_lib, rule):
    _run_steps(gpu_lib, rule, "bf16", N=2, H=3, d=128, steps=2, seed=530, packed_cov=True, normalize_keys=True)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_decode_structured_keys(gpu_lib, rule):
    _run_steps(gpu_lib, rule, "f32", N=2, H=2, d=64, steps=2, seed=700, structured=True)


def test_decode_lambda_zero_is_backbone(gpu_lib):
    """b = -inf: the step equals the plain GLA read o = S_t q (cleaning off exactly)."""
    import torch
    from curvature_conditioned_query_amd import ccq_decode_step as gpu_step
    N, H, d = 2, 3, 64
    carry = _prefix_carry("gla", N, H, d, 20, 900)
    (S, C, m, n), (S64, C64, m64, n64) = up_carry(carry)
    tok = decode_tokens("gla", N, H, d, 901, "f32")
    b = np.full((H,), -np.inf, np.float32)
    o = gpu_step("gla", up(tok["q"]), up(tok["k"]), up(tok["v"]), up(tok["g"]), None,
                 torch.from_numpy(tok["w_lam"]).cuda(), torch.from_numpy(b).cuda(), S, C, m, n)
    torch.cuda.synchronize()
    S_new = S64 * np.exp(tok["g"].astype(np.float64))[:, :, None, :] + \
        tok["v"].astype(np.float64)[..., :, None] * tok["k"].astype(np.float64)[..., None, :]
    ref = np.einsum("nhvk,nhk->nhv", S_new, tok["q"].astype(np.float64))
    assert normwise_error(down(o), ref) <= 1e-5


@pytest.mark.parametrize("packed_cov", [False, True])
@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_decode_full_size_sampled(gpu_lib, rule, packed_cov):
    """The benchmark's decode shape and launch (256 sequences x 16 heads, d = 128, bf16 token,
    fp32 state, n = 8192).  Carries are built on the device and are consistent: 64 unit keys per
    head, each counted 128 times (C = 128 sum k k^T, ksum = 128 sum k, n = 8192), S random.  One
    step runs over every head; sampled heads are checked against the oracle step from the same
    carry values."""
    import torch
    from curvature_conditioned_query_amd import ccq_decode_step as gpu_step
    N, H, d, reps, m_keys = 256, 16, 128, 128, 64
    gen = torch.Generator(device="cuda").manual_seed(4242)
    K = torch.randn((N, H, m_keys, d), generator=gen, device="cuda")
    K = K / K.norm(dim=-1, keepdim=True)
    C = reps * (K.transpose(-1, -2).contiguous() @ K)
    C = ((C + C.transpose(-1, -2)) / 2).contiguous()  # exactly symmetric, as a sum of k k^T is
    m = (reps * K.sum(dim=2)).contiguous()
    n = torch.full((N, H), reps * m_keys, dtype=torch.int64, device="cuda")
    S = (torch.randn((N, H, d, d), generator=gen, device="cuda") / np.sqrt(d)).contiguous()
    del K
    tok = decode_tokens(rule, N, H, d, 4243, "bf16")
    sample = [(0, 0), (255, 15), (100, 7), (31, 3)]
    before = {(i, h): tuple(t[i, h].double().cpu().numpy() for t in (S, C, m)) + (int(n[i, h]),) for i, h in sample}
    if packed_cov:  # the same C as its upper triangle, row by row
        iu = torch.triu_indices(d, d, device="cuda")
        C = C[:, :, iu[0], iu[1]].contiguous()
    o = gpu_step(rule, up(tok["q"], "bf16"), up(tok["k"], "bf16"), up(tok["v"], "bf16"), up(tok["g"], "bf16"),
                 up(tok["beta"], "bf16"), torch.from_numpy(tok["w_lam"]).cuda(),
                 torch.from_numpy(tok["b_lam"]).cuda(), S, C, m, n, packed_cov=packed_cov)
    torch.cuda.synchronize()
    assert bool(torch.all(n == reps * m_keys + 1))
    for (i, h) in sample:
        S0, C0, m0, n0 = before[(i, h)]
        carry = Carry(S0[None, None], C0[None, None], m0[None, None], np.array([[n0]], np.int64))
        pick = lambda a: None if a is None else a[i:i + 1, h:h + 1]  # noqa: E731
        o_ref, ref = ccq_decode_step(pick(tok["q"]), pick(tok["k"]), pick(tok["v"]), pick(tok["g"]),
                                     pick(tok["beta"]), tok["w_lam"][h:h + 1], tok["b_lam"][h:h + 1], rule, carry)
        err = normwise_error(down(o[i:i + 1, h:h + 1]), o_ref)
        print(f"decode full-size {rule} packed={packed_cov} head ({i},{h}): o err {err:.3e}", flush=True)
        assert err <= TOL["bf16"]
        assert normwise_error(down(S[i:i + 1, h:h + 1]), ref.S) <= STATE_TOL
        C_ref = pack_upper(ref.C) if packed_cov else ref.C
        assert normwise_error(down(C[i:i + 1, h:h + 1]), C_ref) <= STATE_TOL
        assert normwise_error(down(m[i:i + 1, h:h + 1])[:, :, :, None], ref.m[:, :, :, None]) <= STATE_TOL


@pytest.mark.parametrize("rule", ["gla", "gdn"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_normalize_keys_flag(gpu_lib, rule, dtype):
    """Raw key (any scale, one all-zero) with the normalise-keys flag == oracle step on the unit key."""
    import torch
    from curvature_conditioned_query_amd import ccq_decode_step as gpu_step
    N, H, d = 3, 2, 128
    carry = _prefix_carry(rule, N, H, d, 29, 901)
    (S, C, m, n), (S64, C64, m64, n64) = up_carry(carry)
    tok = decode_tokens(rule, N, H, d, 902, dtype)
    rng = np.random.default_rng(903)
    k_raw = (tok["k"] * rng.uniform(0.05, 20.0, size=(N, H, 1))).astype(np.float32)
    k_raw[2, 1] = 0.0
    if dtype == "bf16":
        from curvature_conditioned_query_amd.inputs import bf16_round
        k_raw = bf16_round(k_raw)
    o = gpu_step(rule, up(tok["q"], dtype), up(k_raw, dtype), up(tok["v"], dtype), up(tok["g"], dtype),
                 up(tok["beta"], dtype), torch.from_numpy(tok["w_lam"]).cuda(),
                 torch.from_numpy(tok["b_lam"]).cuda(), S, C, m, n, normalize_keys=True)
    torch.cuda.synchronize()
    o_ref, ref = ccq_decode_step(tok["q"], unit_keys(k_raw), tok["v"], tok["g"], tok["beta"], tok["w_lam"],
                                 tok["b_lam"], rule, Carry(S64, C64, m64, n64))
    err = normwise_error(down(o), o_ref)
    print(f"decode normalize-keys {rule} {dtype}: o err {err:.3e}", flush=True)
    assert err <= TOL[dtype]
    # fp32 state: the bf16 key is normalised in fp32 on both sides up to the oracle's fp64
    assert normwise_error(down(C), ref.C) <= (STATE_TOL if dtype == "f32" else 1e-4)
    assert normwise_error(down(S), ref.S) <= (STATE_TOL if dtype == "f32" else 1e-4)

"""Decode-step parity: HIP kernel through the C ABI vs the fp64 oracle."""

import numpy as np
import pytest

from curvature_conditioned_query_amd.inputs import decode_tokens, gdn_inputs, gla_inputs, structured_inputs
from oracle import Carry, ccq_decode_step, ccq_recurrent, normwise_error

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


def _run_steps(gpu_lib, rule, dtype, N, H, d, steps, seed, structured=False):
    import torch
    from curvature_conditioned_query_amd import ccq_decode_step as gpu_step
    carry = _prefix_carry(rule, N, H, d, 37, seed)
    (S, C, m, n), (S64, C64, m64, n64) = up_carry(carry)
    ref = Carry(S64, C64, m64, n64)
    for s in range(steps):
        tok = decode_tokens(rule, N, H, d, seed + 1 + s, dtype)
        if structured:
            sx = structured_inputs(rule, N, H, 1, d, seed + 100 + s, dtype)
            tok.update(k=sx.k[:, :, 0], w_lam=sx.w_lam, b_lam=sx.b_lam)
        o = gpu_step(rule, up(tok["q"], dtype), up(tok["k"], dtype), up(tok["v"], dtype), up(tok["g"], dtype),
                     up(tok["beta"], dtype), torch.from_numpy(tok["w_lam"]).cuda(),
                     torch.from_numpy(tok["b_lam"]).cuda(), S, C, m, n)
        torch.cuda.synchronize()
        o_ref, ref = ccq_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], tok["w_lam"],
                                     tok["b_lam"], rule, ref)
        err = normwise_error(down(o), o_ref)
        print(f"decode {rule} {dtype} d={d} step {s}: o err {err:.3e}", flush=True)
        assert err <= TOL[dtype]
        assert normwise_error(down(S), ref.S) <= STATE_TOL
        assert normwise_error(down(C), ref.C) <= STATE_TOL
        assert normwise_error(down(m)[:, :, :, None], ref.m[:, :, :, None]) <= STATE_TOL
        assert np.array_equal(down(n), ref.n)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_matches_oracle(gpu_lib, rule, dtype, d):
    _run_steps(gpu_lib, rule, dtype, N=3, H=2, d=d, steps=3, seed=500 + d)


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

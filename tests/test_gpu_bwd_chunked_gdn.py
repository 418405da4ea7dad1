"""Chunked backward parity on the Gated DeltaNet rule: ccq_bwd_chunked through the C ABI vs the fp64
oracle (autograd through the per-token recurrence, ``oracle.ccq_sequence_backward``) on the same inputs.

Gradients compared normwise per (b, h) slab (max |x - y| / max |y|): dq, dk, dv, dlog alpha, dbeta,
the gate's parameter gradient of each head (dw_lambda and db_lambda as one slab) and the carry-in
adjoint (dS0, dC0, dksum0); 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""

import numpy as np
import pytest

from curvature_conditioned_query_amd.inputs import bf16_round, gdn_inputs
from oracle import Carry, ccq_recurrent, ccq_sequence_backward, normwise_error

from gpu_util import down, up, up_carry

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
GRADS = ("dq", "dk", "dv", "dg", "dbeta")


def _cotangent(shape, seed, dtype):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def _gate_grad(dw, db):
    return np.concatenate([np.asarray(dw, np.float64), np.asarray(db, np.float64).reshape(-1, 1)], axis=1)


def _run(dtype, B, H, T, d, seed, carry=False, adjoint=False, b_lam=-2.0, slow_decay=False):
    import torch
    from curvature_conditioned_query_amd import ccq_bwd_chunked
    x = gdn_inputs(B, H, T, d, seed, dtype, b_lam=b_lam)
    if slow_decay:  # log alpha ~ -0.005: the state transitions stay O(1) over many chunks
        x.g = (x.g / 16).astype(np.float32)
        if dtype == "bf16":
            x.g = bf16_round(x.g)
    do = _cotangent((B, H, T, d), seed + 1, dtype)
    dev_carry = ref_carry = None
    if carry:  # the carry after a 70-token prefix of other inputs
        pre = gdn_inputs(B, H, 70, d, seed + 2, "f32", b_lam=b_lam)
        _, c = ccq_recurrent(pre.q, pre.k, pre.v, pre.g, pre.beta, x.w_lam, x.b_lam, "gdn")
        dev_carry, (S64, C64, m64, n64) = up_carry(c)
        ref_carry = Carry(S64, C64, m64, n64)
    adj = None
    adj_np = {}
    if adjoint:
        rng = np.random.default_rng(seed + 3)
        adj_np = dict(dS_T=rng.standard_normal((B, H, d, d)).astype(np.float32),
                      dC_T=rng.standard_normal((B, H, d, d)).astype(np.float32) * np.float32(1e-2),
                      dm_T=rng.standard_normal((B, H, d)).astype(np.float32) * np.float32(1e-1))
        adj = tuple(torch.from_numpy(adj_np[k]).cuda() for k in ("dS_T", "dC_T", "dm_T"))
    out = ccq_bwd_chunked("gdn", up(x.q, dtype), up(x.k, dtype), up(x.v, dtype), up(x.g, dtype),
                          torch.from_numpy(x.w_lam).cuda(), torch.from_numpy(x.b_lam).cuda(), up(do, dtype),
                          carry_in=dev_carry, carry_out_adjoint=adj, want_carry_in_adjoint=True,
                          beta=up(x.beta, dtype))
    torch.cuda.synchronize()
    ref = ccq_sequence_backward(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, "gdn", do, carry=ref_carry,
                                **{k: v.astype(np.float64) for k, v in adj_np.items()})
    got = dict(dq=out["dq"], dk=out["dk"], dv=out["dv"], dg=out["dlog_alpha"], dbeta=out["dbeta"], dS=out["dS0"],
               dC=out["dC0"], dm=out["dksum0"])
    errs = {}
    for key in GRADS + ("dS", "dC", "dm"):
        g = down(got[key])
        r = ref[key]
        if g.ndim == 3 and key in ("dg", "dbeta"):  # [B, H, T] per-token scalars: one slab per (b, h)
            g, r = g[..., None], r[..., None]
        if key == "dm":
            g, r = g[..., None], r[..., None]
        errs[key] = normwise_error(g, r)
    errs["dwdb"] = normwise_error(_gate_grad(down(out["dw_lambda"]).sum(axis=0), down(out["db_lambda"]).sum(axis=0)),
                                  _gate_grad(ref["dw"], ref["db"]))
    print(f"gdn bwd {dtype} B={B} H={H} T={T} d={d} carry={carry} adjoint={adjoint}: "
          + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    tol = TOL[dtype]
    for key, e in errs.items():
        assert e <= tol, (key, e)
    return out, ref


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_gdn_bwd_matches_oracle(gpu_lib, dtype, d):
    """Three full chunks and a ragged one, from a zero carry."""
    _run(dtype, B=1, H=2, T=200, d=d, seed=2100 + d)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_gdn_bwd_carry_and_final_adjoint(gpu_lib, dtype, d):
    """From a carry in, with the adjoint of the carry out given: every gradient and the carry-in
    adjoint."""
    _run(dtype, B=2, H=1, T=150, d=d, seed=2200 + d, carry=True, adjoint=True)


@pytest.mark.parametrize("T", [1, 37, 64, 65, 128])
def test_gdn_bwd_short_and_boundary_lengths(gpu_lib, T):
    """One token, a single ragged chunk, exactly one chunk, one chunk plus a token, two chunks."""
    _run("f32", B=1, H=2, T=T, d=64, seed=2300 + T, carry=(T % 2 == 1), adjoint=True)


@pytest.mark.parametrize("B,H,T", [(8, 16, 320), (16, 16, 130), (1, 2, 1000)])
def test_gdn_bwd_multi_chunk_segments(gpu_lib, B, H, T):
    """The carry walk over segments (the segment count follows the number of chains): 128 chains
    give two segments of three and two chunks, 256 chains one segment, 2 chains 16 segments of one
    chunk; with a carry in and a carry-out adjoint."""
    _run("bf16", B=B, H=H, T=T, d=64, seed=2600 + T, carry=True, adjoint=True)


def test_gdn_bwd_slow_decay_segments(gpu_lib):
    """Slow decay (the transitions stay near I over many chunks, so the carried-back adjoint of the
    state reaches far back) across 16 segments, fp32."""
    _run("f32", B=1, H=2, T=1000, d=64, seed=2700, carry=True, adjoint=True, slow_decay=True)


def test_gdn_bwd_gate_off(gpu_lib):
    """b = -inf: the cleaning is off, so dw and db are exactly zero and the rest is the plain Gated
    DeltaNet backward (the oracle with lambda = 0)."""
    out, _ = _run("f32", B=1, H=2, T=130, d=64, seed=2400, b_lam=-np.inf)
    assert np.all(down(out["dw_lambda"]) == 0.0) and np.all(down(out["db_lambda"]) == 0.0)


def test_gdn_bwd_strong_gate(gpu_lib):
    """b = +4 (lambda near 1 everywhere): the statistics' share of dq and dk is large."""
    _run("f32", B=1, H=1, T=140, d=64, seed=2500, b_lam=4.0, carry=True)


def test_gdn_bwd_full_size_sampled(gpu_lib):
    """The Gated DeltaNet prefill shape (B = 4, H = 16, T = 4096, d = 128, bf16, zero carry) in one
    launch; one sampled (b, h) chain against the oracle over all 4096 tokens."""
    import torch
    from curvature_conditioned_query_amd import ccq_bwd_chunked
    B, H, T, d, seed = 4, 16, 4096, 128, 1002
    x = gdn_inputs(B, H, T, d, seed, "bf16")
    do = _cotangent((B, H, T, d), seed + 7, "bf16")
    out = ccq_bwd_chunked("gdn", up(x.q, "bf16"), up(x.k, "bf16"), up(x.v, "bf16"), up(x.g, "bf16"),
                          torch.from_numpy(x.w_lam).cuda(), torch.from_numpy(x.b_lam).cuda(), up(do, "bf16"),
                          beta=up(x.beta, "bf16"))
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dw_lambda", "db_lambda"):
        assert bool(torch.isfinite(out[key]).all()), key
    b, h = 2, 11
    sl = lambda a: a[b:b + 1, h:h + 1]  # noqa: E731
    ref = ccq_sequence_backward(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), x.w_lam[h:h + 1], x.b_lam[h:h + 1],
                                "gdn", sl(do))
    got = dict(dq=out["dq"], dk=out["dk"], dv=out["dv"], dg=out["dlog_alpha"], dbeta=out["dbeta"])
    for key in GRADS:
        g, r = down(got[key][b:b + 1, h:h + 1]), ref[key]
        if key in ("dg", "dbeta"):
            g, r = g[..., None], r[..., None]
        e = normwise_error(g, r)
        print(f"gdn bwd full-size chain ({b},{h}) {key} err {e:.2e}", flush=True)
        assert e <= TOL["bf16"], key
    e = normwise_error(_gate_grad(down(out["dw_lambda"][b, h])[None], down(out["db_lambda"][b, h]).reshape(1)),
                       _gate_grad(ref["dw"], ref["db"]))
    print(f"gdn bwd full-size chain ({b},{h}) dw, db err {e:.2e}", flush=True)
    assert e <= TOL["bf16"]

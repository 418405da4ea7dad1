"""Backward of one recurrence step (the adjoint of the decode step): HIP kernel through the C ABI
vs the fp64 autograd oracle, for one step and chained in reverse over a sequence.

Both sides start from the same stored values (bf16 inputs are exact in fp32) and the kernel
computes in fp32, so the bar is the fp32 one for every gradient, 1e-4 normwise per (b, h) slab
(the longest fp32 sums are d = 128 terms of O(1) products; measured errors are about 1e-6)."""

import numpy as np
import pytest

from curvature_conditioned_query_amd.inputs import decode_tokens, gdn_inputs, gla_inputs
from oracle import Carry, ccq_decode_step, ccq_recurrent, ccq_sequence_backward, ccq_step_backward, normwise_error

from gpu_util import down, up

pytestmark = pytest.mark.gpu

TOL = 1e-4
D = 128


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _gpu_step(rule, dtype, tok, w, b, c, do, dS, dC, dm):
    import torch
    from curvature_conditioned_query_amd import ccq_step_backward as gpu
    dSd, dCd, dmd = _dev(dS), _dev(dC), _dev(dm)
    out = gpu(rule, up(tok["q"], dtype), up(tok["k"], dtype), up(tok["v"], dtype), up(tok["g"], dtype),
              up(tok["beta"], dtype), _dev(w), _dev(b), _dev(c.S), _dev(c.C), _dev(c.m),
              torch.from_numpy(np.asarray(c.n, np.int64)).cuda(), _dev(do), dSd, dCd, dmd)
    torch.cuda.synchronize()
    res = {k: (None if t is None else down(t)) for k, t in out.items()}
    res.update(dS=down(dSd), dC=down(dCd), dm=down(dmd))
    return res


def _carry32(c):
    return Carry(c.S.astype(np.float32).astype(np.float64), c.C.astype(np.float32).astype(np.float64),
                 c.m.astype(np.float32).astype(np.float64), np.asarray(c.n, np.int64))


def _compare(got, ref, rule, tag):
    pairs = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dlog_alpha", "dg"), ("dw_lambda", "dw"), ("dS", "dS"),
             ("dC", "dC"), ("dm", "dm")]
    if rule == "gdn":
        pairs.append(("dbeta", "dbeta"))
    errs = {}
    for gk, rk in pairs:
        x, y = got[gk], ref[rk]
        if x.ndim == 2:
            x, y = x[..., None], y[..., None]
        errs[gk] = normwise_error(x, y)
    eb = np.max(np.abs(got["db_lambda"] - ref["db"])) / max(np.max(np.abs(ref["db"])), 1e-30)
    errs["db_lambda"] = eb
    print(f"{tag}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= TOL, (tag, k, v)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_backward_matches_oracle(rule, dtype):
    N, H = 3, 2
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(N, H, 37, D, 600, "f32", b_lam=0.3)
    _, c = ccq_recurrent(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule)
    c = _carry32(c)
    tok = decode_tokens(rule, N, H, D, 601, dtype)
    w, b = x.w_lam.astype(np.float64), np.full(H, 0.3)
    rng = np.random.default_rng(602)
    do = rng.standard_normal((N, H, D)).astype(np.float32)
    dS = rng.standard_normal((N, H, D, D)).astype(np.float32)
    dC = (rng.standard_normal((N, H, D, D)) * 0.1).astype(np.float32)
    dm = rng.standard_normal((N, H, D)).astype(np.float32)
    ref = ccq_step_backward(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], w, b, rule, c.S, c.C, c.m, c.n,
                            do, dS, dC, dm)
    got = _gpu_step(rule, dtype, tok, w, b, c, do, dS, dC, dm)
    _compare(got, ref, rule, f"step {rule} {dtype}")


def test_step_backward_gate_off():
    """b = -inf: the cleaning is off, so the gate parameters get exactly zero gradient and the
    statistic adjoint passes through unchanged."""
    N, H = 2, 2
    x = gla_inputs(N, H, 20, D, 610, "f32")
    _, c = ccq_recurrent(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, "gla")
    c = _carry32(c)
    tok = decode_tokens("gla", N, H, D, 611, "f32")
    b = np.full(H, -np.inf)
    rng = np.random.default_rng(612)
    do = rng.standard_normal((N, H, D)).astype(np.float32)
    dC = rng.standard_normal((N, H, D, D)).astype(np.float32)
    got = _gpu_step("gla", "f32", tok, x.w_lam, b, c, do, np.zeros((N, H, D, D)), dC, np.zeros((N, H, D)))
    assert np.array_equal(got["dw_lambda"], np.zeros_like(got["dw_lambda"]))
    assert np.array_equal(got["db_lambda"], np.zeros_like(got["db_lambda"]))
    assert np.array_equal(got["dC"], dC.astype(np.float64))
    ref = ccq_step_backward(tok["q"], tok["k"], tok["v"], tok["g"], None, x.w_lam, b, "gla", c.S, c.C, c.m, c.n, do,
                            None, dC.astype(np.float64), None)
    assert normwise_error(got["dq"], ref["dq"]) <= TOL


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_step_backward_chained_over_a_sequence(rule):
    """Backpropagation through 6 tokens: the step kernel run in reverse, each time from that
    token's carry before the step (the oracle's forward carries, rounded to fp32), with the
    state adjoints handed from step to step, against autograd through the whole recurrence."""
    B, H, T = 2, 2, 6
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(B, H, T, D, 620, "bf16", b_lam=0.2)
    rng = np.random.default_rng(621)
    do = rng.standard_normal((B, H, T, D)).astype(np.float32)
    ref = ccq_sequence_backward(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule, do)
    states = [Carry.zeros(B, H, D, D)]
    for t in range(T):
        sl = lambda a: None if a is None else a[:, :, t]  # noqa: E731
        _, c1 = ccq_decode_step(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), x.w_lam, x.b_lam, rule,
                                states[-1].copy())
        states.append(_carry32(c1))
    dS, dC, dm = np.zeros((B, H, D, D)), np.zeros((B, H, D, D)), np.zeros((B, H, D))
    got = {k: np.zeros((B, H, T, D)) for k in ("dq", "dk", "dv")}
    got["dg"] = np.zeros(np.shape(x.g))
    got["dbeta"] = np.zeros((B, H, T))
    dw = np.zeros((H, D))
    for t in reversed(range(T)):
        sl = lambda a: None if a is None else a[:, :, t]  # noqa: E731
        tok = dict(q=sl(x.q), k=sl(x.k), v=sl(x.v), g=sl(x.g), beta=sl(x.beta))
        r = _gpu_step(rule, "bf16", tok, x.w_lam, x.b_lam, states[t], do[:, :, t], dS, dC, dm)
        got["dq"][:, :, t], got["dk"][:, :, t], got["dv"][:, :, t] = r["dq"], r["dk"], r["dv"]
        got["dg"][:, :, t] = r["dlog_alpha"]
        if rule == "gdn":
            got["dbeta"][:, :, t] = r["dbeta"]
        dw += r["dw_lambda"].sum(axis=0)
        dS, dC, dm = r["dS"], r["dC"], r["dm"]
    errs = {k: normwise_error(got[k], ref[k]) for k in ("dq", "dk", "dv")}
    errs["dg"] = normwise_error(got["dg"][..., None] if rule == "gdn" else got["dg"],
                                ref["dg"][..., None] if rule == "gdn" else ref["dg"])
    if rule == "gdn":
        errs["dbeta"] = normwise_error(got["dbeta"][..., None], ref["dbeta"][..., None])
    errs["dw"] = np.max(np.abs(dw - ref["dw"])) / np.max(np.abs(ref["dw"]))
    print(f"sequence {rule}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)


def test_step_backward_full_size_sampled():
    """The decode benchmark's shape (256 sequences x 16 heads, d = 128, bf16 token, fp32 state):
    every head on the GPU, sampled heads against the oracle."""
    import torch
    from curvature_conditioned_query_amd import ccq_step_backward as gpu
    N, H = 256, 16
    gen = torch.Generator(device="cuda").manual_seed(630)
    K = torch.randn((N, H, 32, D), generator=gen, device="cuda")
    K = K / K.norm(dim=-1, keepdim=True)
    C = 64 * (K.transpose(-1, -2).contiguous() @ K)
    C = ((C + C.transpose(-1, -2)) / 2).contiguous()
    m = (64 * K.sum(dim=2)).contiguous()
    del K
    n = torch.full((N, H), 2048, dtype=torch.int64, device="cuda")
    S = (torch.randn((N, H, D, D), generator=gen, device="cuda") / np.sqrt(D)).contiguous()
    dS = torch.randn((N, H, D, D), generator=gen, device="cuda").contiguous()
    dC = (torch.randn((N, H, D, D), generator=gen, device="cuda") * 0.01).contiguous()
    dm = torch.randn((N, H, D), generator=gen, device="cuda").contiguous()
    do = torch.randn((N, H, D), generator=gen, device="cuda").contiguous()
    tok = decode_tokens("gla", N, H, D, 631, "bf16")
    w = torch.from_numpy(tok["w_lam"]).cuda()
    b = torch.full((H,), 0.5, device="cuda")
    sample = [(0, 0), (255, 15), (77, 9)]
    before = {(i, h): tuple(t[i, h].double().cpu().numpy() for t in (S, C, m, dS, dC, dm, do)) for i, h in sample}
    out = gpu("gla", up(tok["q"], "bf16"), up(tok["k"], "bf16"), up(tok["v"], "bf16"), up(tok["g"], "bf16"), None,
              w, b, S, C, m, n, do, dS, dC, dm)
    torch.cuda.synchronize()
    for (i, h) in sample:
        Sx, Cx, mx, dSx, dCx, dmx, dox = before[(i, h)]
        pick = lambda a: a[i:i + 1, h:h + 1]  # noqa: E731
        ref = ccq_step_backward(pick(tok["q"]), pick(tok["k"]), pick(tok["v"]), pick(tok["g"]), None,
                                tok["w_lam"][h:h + 1], np.array([0.5]), "gla", Sx[None, None], Cx[None, None],
                                mx[None, None], np.array([[2048]]), dox[None, None], dSx[None, None],
                                dCx[None, None], dmx[None, None])
        got = {k: (None if t is None else down(t[i:i + 1, h:h + 1])) for k, t in out.items()}
        got.update(dS=down(dS[i:i + 1, h:h + 1]), dC=down(dC[i:i + 1, h:h + 1]), dm=down(dm[i:i + 1, h:h + 1]))
        _compare(got, ref, "gla", f"full size head ({i},{h})")

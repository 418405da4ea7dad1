"""Pins of the gradient oracle (``oracle/grad.py``) against things other than itself: its forward
step against the numpy oracle (a separate implementation of the same definitions), its
gradients against central finite differences of the numpy oracle's forward, the λ = 0 case, and
the chaining of step adjoints in reverse against autograd through a whole sequence (itself
checked by finite differences).  Planted slips in a private copy of the module are caught."""

import os
import types

import numpy as np
import pytest

from curvature_conditioned_query_amd.inputs import decode_tokens, gdn_inputs, gla_inputs
from oracle import Carry, ccq_decode_step, ccq_recurrent, ccq_sequence_backward, ccq_step_backward

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "grad.py")


def _problem(rule, N=2, H=2, d=6, seed=0):
    """A carry after a short prefix, one token, and random cotangents (fp64 numpy)."""
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(N, H, 9, d, seed, "f32", b_lam=0.3)
    _, c = ccq_recurrent(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule)
    tok = decode_tokens(rule, N, H, d, seed + 1, "f32")
    rng = np.random.default_rng(seed + 2)
    cot = dict(do=rng.standard_normal((N, H, d)), dS1=rng.standard_normal((N, H, d, d)),
               dC1=rng.standard_normal((N, H, d, d)), dm1=rng.standard_normal((N, H, d)))
    return c, tok, x.w_lam.astype(np.float64), np.full(H, 0.3), cot


def _loss_numpy(rule, c, tok, w, b, cot):
    o, c1 = ccq_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], w, b, rule, c.copy())
    return (np.sum(o * cot["do"]) + np.sum(c1.S * cot["dS1"]) + np.sum(c1.C * cot["dC1"])
            + np.sum(c1.m * cot["dm1"]))


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_step_forward_matches_numpy_oracle(rule):
    import torch
    from oracle import ccq_step_torch
    c, tok, w, b, _ = _problem(rule)
    T = lambda a: None if a is None else torch.as_tensor(np.asarray(a, np.float64))  # noqa: E731
    o, S1, C1, m1 = ccq_step_torch(T(tok["q"]), T(tok["k"]), T(tok["v"]), T(tok["g"]), T(tok["beta"]), T(w), T(b),
                                   rule, T(c.S), T(c.C), T(c.m), T(c.n.astype(np.float64)))
    o_ref, c1 = ccq_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], w, b, rule, c.copy())
    assert np.allclose(o.numpy(), o_ref, atol=1e-12)
    assert np.allclose(S1.numpy(), c1.S, atol=1e-12)
    assert np.allclose(C1.numpy(), c1.C, atol=1e-12)
    assert np.allclose(m1.numpy(), c1.m, atol=1e-12)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_step_gradients_match_finite_differences(rule):
    c, tok, w, b, cot = _problem(rule, N=1, H=2, d=5, seed=11)
    gr = ccq_step_backward(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], w, b, rule, c.S, c.C, c.m, c.n,
                           cot["do"], cot["dS1"], cot["dC1"], cot["dm1"])
    h = 1e-6
    rng = np.random.default_rng(12)
    # directional derivatives along random directions, one input at a time
    names = ["q", "k", "v", "g"] + (["beta"] if rule == "gdn" else [])
    for nm in names:
        e = rng.standard_normal(np.shape(tok[nm]))
        tp = dict(tok); tp[nm] = tok[nm] + h * e
        tm = dict(tok); tm[nm] = tok[nm] - h * e
        num = (_loss_numpy(rule, c, tp, w, b, cot) - _loss_numpy(rule, c, tm, w, b, cot)) / (2 * h)
        ana = np.sum(gr["d" + nm] * e)
        assert np.isclose(ana, num, rtol=1e-6, atol=1e-8), (nm, ana, num)
    for nm in ["S", "C", "m"]:
        base = getattr(c, nm)
        e = rng.standard_normal(base.shape)
        cp, cm = c.copy(), c.copy()
        setattr(cp, nm, base + h * e)
        setattr(cm, nm, base - h * e)
        num = (_loss_numpy(rule, cp, tok, w, b, cot) - _loss_numpy(rule, cm, tok, w, b, cot)) / (2 * h)
        ana = np.sum(gr["d" + nm] * e)
        assert np.isclose(ana, num, rtol=1e-6, atol=1e-8), (nm, ana, num)
    e = rng.standard_normal(w.shape)
    num = (_loss_numpy(rule, c, tok, w + h * e, b, cot) - _loss_numpy(rule, c, tok, w - h * e, b, cot)) / (2 * h)
    assert np.isclose(np.sum(gr["dw"].sum(axis=0) * e), num, rtol=1e-6, atol=1e-8)
    e = rng.standard_normal(b.shape)
    num = (_loss_numpy(rule, c, tok, w, b + h * e, cot) - _loss_numpy(rule, c, tok, w, b - h * e, cot)) / (2 * h)
    assert np.isclose(np.sum(gr["db"].sum(axis=0) * e), num, rtol=1e-6, atol=1e-8)


def test_step_gradients_gate_off():
    """b = -inf: the cleaning is off exactly, so the gate parameters get no gradient and
    dq = S'^T do."""
    c, tok, w, _, cot = _problem("gla", seed=21)
    b = np.full(2, -np.inf)
    gr = ccq_step_backward(tok["q"], tok["k"], tok["v"], tok["g"], None, w, b, "gla", c.S, c.C, c.m, c.n,
                           cot["do"])
    assert np.array_equal(gr["dw"], np.zeros_like(gr["dw"]))
    assert np.array_equal(gr["db"], np.zeros_like(gr["db"]))
    S1 = c.S * np.exp(tok["g"])[..., None, :] + tok["v"][..., :, None] * tok["k"][..., None, :]
    assert np.allclose(gr["dq"], np.einsum("nhvk,nhv->nhk", S1, cot["do"]), atol=1e-12)
    assert np.array_equal(gr["dC"], np.zeros_like(gr["dC"]))


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_sequence_backward_finite_differences_and_step_chain(rule):
    """Autograd through T = 4 tokens against finite differences of the numpy recurrence, and the
    step adjoints chained in reverse (states from the forward steps) against it."""
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(1, 2, 4, 5, 31, "f32", b_lam=0.2)
    rng = np.random.default_rng(32)
    do = rng.standard_normal((1, 2, 4, 5))
    seq = ccq_sequence_backward(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule, do)

    def loss(xx):
        o, _ = ccq_recurrent(xx.q, xx.k, xx.v, xx.g, xx.beta, xx.w_lam, xx.b_lam, rule)
        return np.sum(o * do)

    h = 1e-6
    for nm in ["q", "k", "v", "g"] + (["beta"] if rule == "gdn" else []) + ["w_lam"]:
        e = rng.standard_normal(np.shape(getattr(x, nm)))
        xp = gen(1, 2, 4, 5, 31, "f32", b_lam=0.2)
        xm = gen(1, 2, 4, 5, 31, "f32", b_lam=0.2)
        setattr(xp, nm, getattr(x, nm).astype(np.float64) + h * e)
        setattr(xm, nm, getattr(x, nm).astype(np.float64) - h * e)
        num = (loss(xp) - loss(xm)) / (2 * h)
        key = "dw" if nm == "w_lam" else "d" + nm
        assert np.isclose(np.sum(seq[key] * e), num, rtol=1e-6, atol=1e-8), (nm,)
    # chain the step adjoints backward
    states = [Carry.zeros(1, 2, 5, 5)]
    for t in range(4):
        sl = lambda a: None if a is None else a[:, :, t]  # noqa: E731
        _, c1 = ccq_decode_step(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), x.w_lam, x.b_lam, rule,
                                states[-1].copy())
        states.append(c1)
    dS, dC, dm = (np.zeros((1, 2, 5, 5)), np.zeros((1, 2, 5, 5)), np.zeros((1, 2, 5)))
    acc = {k: np.zeros(np.shape(getattr(x, k if k != "w" else "w_lam"))) for k in ("q", "k", "v", "g")}
    dw = np.zeros((2, 5))
    for t in reversed(range(4)):
        c = states[t]
        sl = lambda a: None if a is None else a[:, :, t]  # noqa: E731
        gr = ccq_step_backward(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), x.w_lam, x.b_lam, rule, c.S, c.C, c.m,
                               c.n, do[:, :, t], dS, dC, dm)
        for k in ("q", "k", "v", "g"):
            acc[k][:, :, t] = gr["d" + k]
        dw += gr["dw"].sum(axis=0)
        dS, dC, dm = gr["dS"], gr["dC"], gr["dm"]
    for k in ("q", "k", "v", "g"):
        assert np.allclose(acc[k], seq["d" + k], atol=1e-10), k
    assert np.allclose(dw, seq["dw"], atol=1e-10)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_sequence_backward_carry_adjoints(rule):
    """With a carry in and the adjoint of the carry out given: the gradients against central
    finite differences of the numpy recurrence with the terms <dS_T, S_T> + <dC_T, C_T> +
    <dm_T, m_T> in the loss (inputs and carry in), and the whole sequence against its two
    halves chained (the second half's carry-in adjoint is the first half's carry-out adjoint)."""
    gen = gla_inputs if rule == "gla" else gdn_inputs
    B, H, T, d = 1, 2, 6, 4
    x = gen(B, H, T, d, 51, "f32", b_lam=0.4)
    pre = gen(B, H, 5, d, 52, "f32", b_lam=0.4)
    _, carry = ccq_recurrent(pre.q, pre.k, pre.v, pre.g, pre.beta, x.w_lam, x.b_lam, rule)
    rng = np.random.default_rng(53)
    do = rng.standard_normal((B, H, T, d))
    adj = dict(dS_T=rng.standard_normal((B, H, d, d)), dC_T=rng.standard_normal((B, H, d, d)),
               dm_T=rng.standard_normal((B, H, d)))
    seq = ccq_sequence_backward(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule, do, carry=carry, **adj)

    def loss(xx, c):
        o, c1 = ccq_recurrent(xx.q, xx.k, xx.v, xx.g, xx.beta, xx.w_lam, xx.b_lam, rule, carry=c.copy())
        return (np.sum(o * do) + np.sum(c1.S * adj["dS_T"]) + np.sum(c1.C * adj["dC_T"])
                + np.sum(c1.m * adj["dm_T"]))

    h = 1e-6
    for nm in ["q", "k", "v", "g", "w_lam", "b_lam"] + (["beta"] if rule == "gdn" else []):
        e = rng.standard_normal(np.shape(getattr(x, nm)))
        xp, xm = gen(B, H, T, d, 51, "f32", b_lam=0.4), gen(B, H, T, d, 51, "f32", b_lam=0.4)
        setattr(xp, nm, getattr(x, nm).astype(np.float64) + h * e)
        setattr(xm, nm, getattr(x, nm).astype(np.float64) - h * e)
        num = (loss(xp, carry) - loss(xm, carry)) / (2 * h)
        key = {"w_lam": "dw", "b_lam": "db"}.get(nm, "d" + nm)
        assert np.isclose(np.sum(seq[key] * e), num, rtol=1e-6, atol=1e-8), (nm,)
    for nm, key in (("S", "dS"), ("C", "dC"), ("m", "dm")):
        e = rng.standard_normal(np.shape(getattr(carry, nm)))
        cp, cm = carry.copy(), carry.copy()
        setattr(cp, nm, getattr(carry, nm) + h * e)
        setattr(cm, nm, getattr(carry, nm) - h * e)
        num = (loss(x, cp) - loss(x, cm)) / (2 * h)
        assert np.isclose(np.sum(seq[key] * e), num, rtol=1e-6, atol=1e-8), (nm,)
    # two halves chained: tokens 3..5 from the carry after tokens 0..2, then tokens 0..2
    sl = lambda a, lo, hi: None if a is None else a[:, :, lo:hi]  # noqa: E731
    _, mid = ccq_recurrent(sl(x.q, 0, 3), sl(x.k, 0, 3), sl(x.v, 0, 3), sl(x.g, 0, 3), sl(x.beta, 0, 3),
                           x.w_lam, x.b_lam, rule, carry=carry.copy())
    second = ccq_sequence_backward(sl(x.q, 3, 6), sl(x.k, 3, 6), sl(x.v, 3, 6), sl(x.g, 3, 6), sl(x.beta, 3, 6),
                                   x.w_lam, x.b_lam, rule, do[:, :, 3:], carry=mid, **adj)
    first = ccq_sequence_backward(sl(x.q, 0, 3), sl(x.k, 0, 3), sl(x.v, 0, 3), sl(x.g, 0, 3), sl(x.beta, 0, 3),
                                  x.w_lam, x.b_lam, rule, do[:, :, :3], carry=carry, dS_T=second["dS"],
                                  dC_T=second["dC"], dm_T=second["dm"])
    for key in ("dq", "dk", "dv", "dg") + (("dbeta",) if rule == "gdn" else ()):
        assert np.allclose(np.concatenate([first[key], second[key]], axis=2), seq[key], atol=1e-10), key
    for key in ("dw", "db"):
        assert np.allclose(first[key] + second[key], seq[key], atol=1e-10), key
    for key in ("dS", "dC", "dm"):
        assert np.allclose(first[key], seq[key], atol=1e-10), key


MUTATIONS = {
    "gla_decay_inverted": ("S1 = S * torch.exp(g)[..., None, :]", "S1 = S * torch.exp(-g)[..., None, :]"),
    "no_count_normalisation": ("u = Cq / n1[..., None]", "u = Cq"),
    "gate_on_key": ("lam = torch.sigmoid((q * w).sum(-1) + b)", "lam = torch.sigmoid((k * w).sum(-1) + b)"),
    "gdn_beta_missing": ("+ beta[..., None, None] * v[..., :, None] * k[..., None, :]",
                         "+ v[..., :, None] * k[..., None, :]"),
}


def _mutant(name):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType(f"grad_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _forward_pin_holds(mod) -> bool:
    import torch
    try:
        for rule in ("gla", "gdn"):
            c, tok, w, b, _ = _problem(rule, seed=41)
            T = lambda a: None if a is None else torch.as_tensor(np.asarray(a, np.float64))  # noqa: E731
            o, S1, _, _ = mod.ccq_step_torch(T(tok["q"]), T(tok["k"]), T(tok["v"]), T(tok["g"]), T(tok["beta"]),
                                             T(w), T(b), rule, T(c.S), T(c.C), T(c.m), T(c.n.astype(np.float64)))
            o_ref, c1 = ccq_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"], w, b, rule, c.copy())
            if not (np.allclose(o.numpy(), o_ref, atol=1e-10) and np.allclose(S1.numpy(), c1.S, atol=1e-10)):
                return False
        return True
    except Exception:
        return False


def test_unmutated_grad_oracle_passes():
    import oracle.grad as real
    assert _forward_pin_holds(real)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_grad_mutation_is_caught(name):
    assert not _forward_pin_holds(_mutant(name))

"""Plain fp64 CPU reference of the gradients of the CCQ recurrence (test infrastructure only;
nothing in the product path imports it).

The pages train the CCQ models from scratch (10100.com write-up, sections "方法解析" point 3
and "代价与边界"), so the read step needs its backward pass.  Here the forward step is written
out once more in plain PyTorch fp64 ops from the same definitions as ``ccq.py`` (the cleaning,
gate and read of the gist.science summary §2 "机制" / "集成", the statistics of §2
"理论推导", the GLA and Gated DeltaNet write rules), and its gradients come from
torch.autograd, the library step of this reference.  It is pinned against the numpy oracle's
forward values and against central finite differences (``tests/test_oracle_grad_pins.py``).

One step, carry (S, C, m, n) -> (S', C', m', n + 1), token (q, k, v, g, beta), gate (w, b):
    C' = C + k k^T,  m' = m + k,  n' = n + 1
    u  = C' q / n' - m' (m' . q) / n'^2,   lam = sigmoid(w . q + b),   q~ = q - lam u
    GLA: S' = S diag(exp g) + v k^T;   GDN: S' = a S (I - beta k k^T) + beta v k^T, a = exp g
    o  = S' q~
The step's backward takes the output gradient do and the adjoint of the carry after the step
(dS', dC', dm') and returns the gradients of every input, including the carry before it.
"""

from __future__ import annotations

import numpy as np
import torch

__all__ = ["ccq_step_torch", "ccq_step_backward", "ccq_sequence_backward"]

f64 = torch.float64


def _t(x):
    return None if x is None else torch.as_tensor(np.asarray(x, dtype=np.float64), dtype=f64)


def ccq_step_torch(q, k, v, g, beta, w, b, rule: str, S, C, m, n):
    """One recurrence step on torch fp64 tensors with leading dims [N, H].
    q, k [N,H,d]; v [N,H,dv]; g GLA [N,H,d] / GDN [N,H]; beta GDN [N,H]; w [H,d]; b [H];
    S [N,H,dv,d]; C [N,H,d,d]; m [N,H,d]; n [N,H] (float).  Returns o, S', C', m'."""
    n1 = n + 1.0
    C1 = C + k[..., :, None] * k[..., None, :]
    m1 = m + k
    Cq = (C1 @ q[..., :, None])[..., 0]
    u = Cq / n1[..., None] - m1 * ((m1 * q).sum(-1) / (n1 * n1))[..., None]
    lam = torch.sigmoid((q * w).sum(-1) + b)
    qc = q - lam[..., None] * u
    if rule == "gla":
        S1 = S * torch.exp(g)[..., None, :] + v[..., :, None] * k[..., None, :]
    elif rule == "gdn":
        a = torch.exp(g)
        Sk = (S @ k[..., :, None])[..., 0]
        S1 = a[..., None, None] * (S - beta[..., None, None] * Sk[..., :, None] * k[..., None, :]) \
            + beta[..., None, None] * v[..., :, None] * k[..., None, :]
    else:
        raise ValueError(rule)
    o = (S1 @ qc[..., :, None])[..., 0]
    return o, S1, C1, m1


def ccq_step_backward(q, k, v, g, beta, w_lam, b_lam, rule: str, S, C, m, n, do, dS1=None, dC1=None,
                      dm1=None):
    """Gradients of L = <do, o> + <dS1, S'> + <dC1, C'> + <dm1, m'> for one step (numpy in,
    numpy out, fp64).  Returns a dict with dq, dk, dv, dg, dbeta (GDN), dw [N,H,d] and db [N,H]
    (per sequence: the per-head parameter gradient is their sum over sequences), and dS, dC, dm
    (the adjoint of the carry before the step)."""
    N, H, d = np.asarray(q).shape
    ins = dict(q=_t(q), k=_t(k), v=_t(v), g=_t(g), beta=_t(beta), S=_t(S), C=_t(C), m=_t(m))
    # per-sequence copies of the gate parameters give per-sequence parameter gradients
    ins["w"] = _t(np.broadcast_to(np.asarray(w_lam, dtype=np.float64), (N, H, d)).copy())
    ins["b"] = _t(np.broadcast_to(np.asarray(b_lam, dtype=np.float64), (N, H)).copy())
    for t in ins.values():
        if t is not None:
            t.requires_grad_(True)
    nn = _t(np.asarray(n, dtype=np.float64))
    o, S1, C1, m1 = ccq_step_torch(ins["q"], ins["k"], ins["v"], ins["g"], ins["beta"], ins["w"], ins["b"], rule,
                                   ins["S"], ins["C"], ins["m"], nn)
    L = (o * _t(do)).sum()
    if dS1 is not None:
        L = L + (S1 * _t(dS1)).sum()
    if dC1 is not None:
        L = L + (C1 * _t(dC1)).sum()
    if dm1 is not None:
        L = L + (m1 * _t(dm1)).sum()
    keys = [kk for kk, t in ins.items() if t is not None]
    grads = torch.autograd.grad(L, [ins[kk] for kk in keys], allow_unused=True)
    out = {}
    for kk, gr in zip(keys, grads):
        out["d" + kk] = np.zeros(ins[kk].shape) if gr is None else gr.detach().numpy()
    return out


def ccq_sequence_backward(q, k, v, g, beta, w_lam, b_lam, rule: str, do, carry=None, dS_T=None, dC_T=None,
                          dm_T=None):
    """Gradients of L = <do, o> + <dS_T, S_T> + <dC_T, C_T> + <dm_T, m_T> through the whole
    recurrence over T tokens (inputs [B,H,T,...], numpy, fp64; the last three terms are present
    when the adjoint of the carry after the last token is given, [B,H,...] each): dq, dk, dv, dg,
    dbeta (GDN), dw [H,d], db [H], and the adjoint of the carry in (dS, dC, dm; of the zero carry
    when none is given).  The reference for chaining the step backward in reverse and for the
    chunked backward."""
    q, k, v, g, do = (_t(x) for x in (q, k, v, g, do))
    beta = _t(beta)
    w = _t(w_lam)
    b = _t(b_lam)
    B, H, T, d = q.shape
    dv_ = v.shape[-1]
    if carry is None:
        S = torch.zeros((B, H, dv_, d), dtype=f64)
        C = torch.zeros((B, H, d, d), dtype=f64)
        m = torch.zeros((B, H, d), dtype=f64)
        n = torch.zeros((B, H), dtype=f64)
    else:
        S, C, m = _t(carry.S), _t(carry.C), _t(carry.m)
        n = _t(np.asarray(carry.n, dtype=np.float64))
    leaves = dict(q=q, k=k, v=v, g=g, beta=beta, w=w, b=b, S=S, C=C, m=m)
    for t in leaves.values():
        if t is not None:
            t.requires_grad_(True)
    St, Ct, mt, nt = S, C, m, n
    L = torch.zeros((), dtype=f64)
    for t in range(T):
        bt = None if beta is None else beta[:, :, t]
        o, St, Ct, mt = ccq_step_torch(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], bt, w, b, rule, St, Ct, mt, nt)
        nt = nt + 1.0
        L = L + (o * do[:, :, t]).sum()
    for adj, state in ((dS_T, St), (dC_T, Ct), (dm_T, mt)):
        if adj is not None:
            L = L + (state * _t(adj)).sum()
    keys = [kk for kk, t in leaves.items() if t is not None]
    grads = torch.autograd.grad(L, [leaves[kk] for kk in keys], allow_unused=True)
    return {"d" + kk: (np.zeros(leaves[kk].shape) if gr is None else gr.detach().numpy())
            for kk, gr in zip(keys, grads)}

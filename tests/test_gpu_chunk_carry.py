"""The chunk carries a prefill writes for the chunked backward (ccq_fwd_params.chunk_carry): each
one against the oracle's carry at that chunk start, and the backward that reads them
(ccq_bwd_params.chunk_carry) against the oracle's gradients, for both write rules, every prefill
kernel (d = 64 fp32 and bf16, the pipelined d = 128 bf16 kernel, the single-role d = 128 kernel
with in-kernel key normalisation), with and without a carry in and at several segment counts."""

import numpy as np
import pytest

from curvature_conditioned_query_amd.inputs import bf16_round, gdn_inputs, gla_inputs
from oracle import Carry, ccq_recurrent, ccq_sequence_backward, normwise_error, unit_keys

from gpu_util import down, up, up_carry

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _oracle_chunk_carries(x, rule, carry, keys):
    """The oracle's carry at every 64-token chunk start: chunk 0's is the carry in (or zeros), each
    later one the recurrence continued over the chunk before it."""
    B, H, T, d = x.q.shape
    c = carry.copy() if carry is not None else Carry.zeros(B, H, d, d)
    out = []
    for ch in range((T + 63) // 64):
        out.append(c.copy())
        sl = slice(64 * ch, min(T, 64 * ch + 64))
        beta = None if x.beta is None else x.beta[:, :, sl]
        _, c = ccq_recurrent(x.q[:, :, sl], keys[:, :, sl], x.v[:, :, sl], x.g[:, :, sl], beta, x.w_lam, x.b_lam,
                             rule, carry=c)
    return out


def _split(buf, B, H, T, d, dtype):
    """The chunk-carry buffer as (S_c, C_c [B, H, NC, d, d], m_c [B, H, NC, d]) host arrays."""
    import torch
    NC = (T + 63) // 64
    E = 2 if dtype == "bf16" else 4
    nmat = B * H * NC * 2 * d * d
    mat = buf[: nmat * E].view(torch.bfloat16 if dtype == "bf16" else torch.float32)
    mat = mat.float().cpu().numpy().astype(np.float64).reshape(B, H, NC, 2, d, d)
    km = buf[nmat * E: nmat * E + B * H * NC * d * 4].view(torch.float32).cpu().numpy().astype(np.float64)
    return mat[:, :, :, 0], mat[:, :, :, 1], km.reshape(B, H, NC, d)


def _case(rule, dtype, d, T, seed, carry=False, segments=0, normalize=False, backward=True):
    import torch
    from curvature_conditioned_query_amd import ccq_bwd_chunked, ccq_fwd_chunked, new_chunk_carry
    B, H = 1, 2
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(B, H, T, d, seed, dtype)
    keys = x.k
    if normalize:  # raw keys of varied length; the kernel (and the oracle) normalise them
        scale = np.random.default_rng(seed + 7).uniform(0.5, 2.0, size=x.k.shape[:-1] + (1,)).astype(np.float32)
        x.k = (x.k * scale).astype(np.float32)
        if dtype == "bf16":
            x.k = bf16_round(x.k)
        keys = unit_keys(x.k)
    dev_carry = ref_carry = None
    if carry:  # the carry after a 70-token prefix of other inputs
        pre = gen(B, H, 70, d, seed + 2, "f32")
        _, c = ccq_recurrent(pre.q, pre.k, pre.v, pre.g, pre.beta, x.w_lam, x.b_lam, rule)
        dev_carry, (S64, C64, m64, n64) = up_carry(c)
        ref_carry = Carry(S64, C64, m64, n64)
    q, k, v, g = up(x.q, dtype), up(x.k, dtype), up(x.v, dtype), up(x.g, dtype)
    beta = up(x.beta, dtype) if x.beta is not None else None
    w, b = torch.from_numpy(x.w_lam).cuda(), torch.from_numpy(x.b_lam).cuda()
    buf = new_chunk_carry(q)
    ccq_fwd_chunked(rule, q, k, v, g, beta, w, b, carry_in=dev_carry, segments=segments, chunk_carry=buf,
                    normalize_keys=normalize)
    torch.cuda.synchronize()
    S_c, C_c, m_c = _split(buf, B, H, T, d, dtype)
    ref = _oracle_chunk_carries(x, rule, ref_carry, keys)
    tol = TOL[dtype]
    worst = 0.0
    for ch, rc in enumerate(ref):
        if ch == 0 and ref_carry is None:  # the empty carry: exactly zero
            assert not S_c[:, :, 0].any() and not C_c[:, :, 0].any() and not m_c[:, :, 0].any()
            continue
        e = max(normwise_error(S_c[:, :, ch], rc.S), normwise_error(C_c[:, :, ch], rc.C),
                normwise_error(m_c[:, :, ch], rc.m))
        worst = max(worst, e)
        assert e <= tol, (ch, e)
    print(f"chunk carries {rule} {dtype} d={d} T={T} carry={carry} segments={segments} normalize={normalize}: "
          f"worst {worst:.2e}", flush=True)
    if not backward:
        return
    do = np.random.default_rng(seed + 1).standard_normal((B, H, T, d)).astype(np.float32)
    if dtype == "bf16":
        do = bf16_round(do)
    out = ccq_bwd_chunked(rule, q, k, v, g, w, b, up(do, dtype), carry_in=dev_carry, want_carry_in_adjoint=True,
                          beta=beta, chunk_carry=buf)
    torch.cuda.synchronize()
    refg = ccq_sequence_backward(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule, do, carry=ref_carry)
    got = dict(dq=out["dq"], dk=out["dk"], dv=out["dv"], dg=out["dlog_alpha"], dS=out["dS0"], dC=out["dC0"],
               dm=out["dksum0"])
    if rule == "gdn":
        got["dbeta"] = out["dbeta"]
    errs = {}
    for key, t in got.items():
        gv, rv = down(t), refg[key]
        if gv.ndim == 3 and key in ("dg", "dbeta", "dm"):
            gv, rv = gv[..., None], rv[..., None]
        errs[key] = normwise_error(gv, rv)
    print("  backward from them: " + " ".join(f"{kk} {vv:.2e}" for kk, vv in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= tol, (key, e)


@pytest.mark.parametrize("rule,dtype,d", [("gla", "f32", 64), ("gla", "bf16", 64), ("gla", "bf16", 128),
                                          ("gdn", "f32", 64), ("gdn", "bf16", 128)])
@pytest.mark.parametrize("carry", [False, True])
def test_chunk_carries_and_backward(gpu_lib, rule, dtype, d, carry):
    """Three full chunks and a ragged one (one segment per chunk at this size)."""
    _case(rule, dtype, d, T=200, seed=4100 + d + (50 if rule == "gdn" else 0), carry=carry)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
@pytest.mark.parametrize("segments", [1, 3])
def test_chunk_carries_across_segments(gpu_lib, rule, segments):
    """Segments of several chunks (each writes its own chunks' carries from its own carry-in)."""
    _case(rule, "bf16", 128, T=600, seed=4200 + segments, carry=True, segments=segments)


def test_chunk_carries_with_key_normalisation(gpu_lib):
    """The single-role GLA kernel at d = 128 (picked for in-kernel key normalisation) writes the carries
    of the normalised keys."""
    _case("gla", "bf16", 128, T=200, seed=4300, normalize=True, backward=False)

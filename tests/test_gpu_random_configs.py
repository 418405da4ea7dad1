"""Seeded sweep of prefill configurations inside the documented limits, each against the oracle.

Every case draws the rule (GLA, Gated DeltaNet), the input dtype (fp32 at d = 64, bf16 at
d = 64 or 128), B, H, a ragged T, the segment count (0 = the library's choice), an optional
carry in (the oracle's fp32-rounded carry after a prefix of its own), the packed-statistics flag
and the normalise-keys flag (raw keys at random scales on the GPU, unit keys for the oracle),
then checks o and the final carry at the bar the inputs' precision sets.  The draws are fixed
by the seed, so a failure names a reproducible case.
"""

import numpy as np
import pytest

from curvature_conditioned_query_amd.inputs import bf16_round, gdn_inputs, gla_inputs
from oracle import Carry, unit_keys

from gpu_util import up_carry
from test_gpu_prefill import check, gpu_prefill, oracle

pytestmark = pytest.mark.gpu


def _configs(n: int, seed: int):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ("f32", "bf16")[int(rng.integers(2))]
        out.append(dict(
            i=i,
            rule=("gla", "gdn")[int(rng.integers(2))],
            dtype=dtype,
            d=64 if dtype == "f32" else int(rng.choice([64, 128])),
            B=int(rng.integers(1, 3)),
            H=int(rng.integers(1, 4)),
            T=int(rng.integers(1, 400)),
            segments=int(rng.integers(0, 7)),
            prefix=int(rng.integers(1, 150)) if rng.random() < 0.5 else 0,
            packed=bool(rng.random() < 0.3),
            normalize=bool(rng.random() < 0.3),
            seed=int(rng.integers(1 << 30)),
        ))
    return out


def _case_id(c):
    flags = ("P" if c["packed"] else "") + ("N" if c["normalize"] else "") + ("C" if c["prefix"] else "")
    return f"{c['i']}-{c['rule']}-{c['dtype']}-d{c['d']}-B{c['B']}H{c['H']}T{c['T']}-s{c['segments']}-{flags or 'x'}"


@pytest.mark.parametrize("cfg", _configs(24, 20261202), ids=_case_id)
def test_random_prefill_config(cfg):
    gen = gla_inputs if cfg["rule"] == "gla" else gdn_inputs
    shape = (cfg["B"], cfg["H"], cfg["T"], cfg["d"])
    x = gen(*shape, cfg["seed"], cfg["dtype"])
    carry = None
    if cfg["prefix"]:
        x0 = gen(cfg["B"], cfg["H"], cfg["prefix"], cfg["d"], cfg["seed"] + 1, "f32")
        _, pre = oracle(x0)
        _, (S, C, m, n) = up_carry(pre)
        carry = Carry(S, C, m, n)
    xr = x
    if cfg["normalize"]:
        rng = np.random.default_rng(cfg["seed"] + 2)
        k_raw = x.k * rng.uniform(0.05, 20.0, size=x.k.shape[:-1] + (1,)).astype(np.float32)
        if cfg["dtype"] == "bf16":
            k_raw = bf16_round(k_raw)
        xr = gen(*shape, cfg["seed"], cfg["dtype"])
        xr.k = unit_keys(k_raw)
        x.k = k_raw
    o, c = gpu_prefill(x, segments=cfg["segments"], carry=carry, packed_cov=cfg["packed"],
                       normalize_keys=cfg["normalize"])
    o_ref, c_ref = oracle(xr, carry)
    check(x, o, c, o_ref, c_ref, tag=f"random {_case_id(cfg)}")


def _decode_configs(n: int, seed: int):
    rng = np.random.default_rng(seed)
    return [dict(i=i, rule=("gla", "gdn")[int(rng.integers(2))], dtype=("f32", "bf16")[int(rng.integers(2))],
                 d=int(rng.choice([64, 128])), N=int(rng.integers(1, 6)), H=int(rng.integers(1, 5)),
                 steps=int(rng.integers(1, 4)), packed=bool(rng.random() < 0.4),
                 normalize=bool(rng.random() < 0.4), seed=int(rng.integers(1 << 30))) for i in range(n)]


@pytest.mark.parametrize("cfg", _decode_configs(12, 20261203),
                         ids=lambda c: f"{c['i']}-{c['rule']}-{c['dtype']}-d{c['d']}-N{c['N']}H{c['H']}-"
                                       f"x{c['steps']}-{'P' if c['packed'] else ''}{'N' if c['normalize'] else ''}")
def test_random_decode_config(gpu_lib, cfg):
    """Decode steps from a prefix carry with random shapes and flags, each step against the oracle."""
    from test_gpu_decode import _run_steps
    _run_steps(gpu_lib, cfg["rule"], cfg["dtype"], cfg["N"], cfg["H"], cfg["d"], cfg["steps"], cfg["seed"],
               packed_cov=cfg["packed"], normalize_keys=cfg["normalize"])


def _bwd_configs(n: int, seed: int):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype, d = [("f32", 64), ("bf16", 64), ("bf16", 128)][i % 3]  # every combination is covered
        out.append(dict(i=i, dtype=dtype, d=d, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                        T=int(rng.integers(1, 300)), carry=bool(rng.random() < 0.5),
                        adjoint=bool(rng.random() < 0.5), b_lam=float(rng.choice([-2.0, 0.0, 2.0])),
                        seed=int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("cfg", _bwd_configs(8, 20261204),
                         ids=lambda c: f"{c['i']}-{c['dtype']}-d{c['d']}-B{c['B']}H{c['H']}T{c['T']}-"
                                       f"{'C' if c['carry'] else ''}{'A' if c['adjoint'] else ''}b{c['b_lam']:+.0f}")
def test_random_bwd_chunked_config(gpu_lib, cfg):
    """The chunked GLA backward with random shapes, carry in, carry-out adjoint and gate bias,
    every gradient against fp64 autograd of the recurrence."""
    from test_gpu_bwd_chunked import _run
    _run(cfg["dtype"], cfg["B"], cfg["H"], cfg["T"], cfg["d"], cfg["seed"], carry=cfg["carry"],
         adjoint=cfg["adjoint"], b_lam=cfg["b_lam"])

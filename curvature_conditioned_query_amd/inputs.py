"""Seeded synthetic inputs for the CCQ read step.

This module only draws random numbers, normalises keys and rounds to the
storage dtype.  It holds none of the method's arithmetic (no statistics, no
gate evaluation, no write rule), so both the HIP path and the CPU oracle can
take their inputs from it without sharing any computation.

Recipe (all draws fp32 from ``numpy.random.default_rng(seed)``, in this order:
q, k, v, gate draws, W_lambda):

* q, v ~ N(0, 1); k ~ N(0, 1) then L2-normalised per token in fp32.  The pages
  require unit keys for the stability bound of the cleaning operator (10100.com
  write-up, section "方法解析", point 2), and the caller is the one that
  normalises them.
* GLA: log alpha = logsigmoid(x) / 16 with x ~ N(0, 1) per key channel.
* Gated DeltaNet: log alpha = -softplus(x) / 8 and beta = sigmoid(y) with
  x, y ~ N(0, 1) per (token, head).
* W_lambda ~ N(0, 1/d_k) (variance 1/d_k); b_lambda = -2 for every head.
* bf16 workloads round every per-token tensor to bf16 (round to nearest even);
  W_lambda and b_lambda stay fp32.

Arrays are returned as fp32 whose values are exactly representable in the
workload dtype, so uploading them with ``tensor.to(torch.bfloat16)`` is exact.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "PrefillInputs",
    "bf16_round",
    "bf16_bits",
    "gla_inputs",
    "gdn_inputs",
    "structured_inputs",
    "decode_tokens",
    "subspace_keys",
    "WORKLOADS",
    "workload_inputs",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, returned as fp32."""
    bits = bf16_bits(x).astype(np.uint32) << 16
    return bits.view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def _unit_rows(x: np.ndarray) -> np.ndarray:
    # generator step: L2-normalise each key row in fp32
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    return (-np.logaddexp(np.float32(0.0), -x)).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (0.5 * (1.0 + np.tanh(0.5 * x))).astype(np.float32)


@dataclasses.dataclass
class PrefillInputs:
    """One prefill workload: per-token tensors [B, H, T, d] (fp32 storage)."""

    rule: str  # "gla" or "gdn"
    dtype: str  # "f32" or "bf16": the dtype q, k, v, gates and o are stored in
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray  # log alpha: GLA [B,H,T,d_k]; GDN [B,H,T]
    beta: Optional[np.ndarray]  # GDN [B,H,T]; GLA None
    w_lam: np.ndarray  # [H, d_k] fp32
    b_lam: np.ndarray  # [H] fp32

    @property
    def shape(self):
        B, H, T, dk = self.q.shape
        return B, H, T, dk, self.v.shape[-1]

    def slab(self, b: int, h: int, t0: int = 0, t1: Optional[int] = None) -> "PrefillInputs":
        """A [1,1,t1-t0,d] view of one (batch, head) chain, for sampled checks."""
        sl = (slice(b, b + 1), slice(h, h + 1), slice(t0, t1))
        return PrefillInputs(
            self.rule, self.dtype, self.q[sl], self.k[sl], self.v[sl], self.g[sl],
            None if self.beta is None else self.beta[sl],
            self.w_lam[h:h + 1], self.b_lam[h:h + 1])


def gla_inputs(B: int, H: int, T: int, d: int, seed: int, dtype: str = "bf16",
               b_lam: float = -2.0, d_v: Optional[int] = None) -> PrefillInputs:
    d_v = d if d_v is None else d_v
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, d), dtype=np.float32)
    k = _unit_rows(rng.standard_normal((B, H, T, d), dtype=np.float32))
    v = rng.standard_normal((B, H, T, d_v), dtype=np.float32)
    x = rng.standard_normal((B, H, T, d), dtype=np.float32)
    w = rng.standard_normal((H, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    g = _logsigmoid(x) / np.float32(16.0)
    return PrefillInputs("gla", dtype, _store(q, dtype), _store(k, dtype), _store(v, dtype),
                         _store(g, dtype), None, w.astype(np.float32),
                         np.full((H,), b_lam, dtype=np.float32))


def gdn_inputs(B: int, H: int, T: int, d: int, seed: int, dtype: str = "bf16",
               b_lam: float = -2.0, d_v: Optional[int] = None) -> PrefillInputs:
    d_v = d if d_v is None else d_v
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, d), dtype=np.float32)
    k = _unit_rows(rng.standard_normal((B, H, T, d), dtype=np.float32))
    v = rng.standard_normal((B, H, T, d_v), dtype=np.float32)
    x = rng.standard_normal((B, H, T), dtype=np.float32)
    y = rng.standard_normal((B, H, T), dtype=np.float32)
    w = rng.standard_normal((H, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    g = -_softplus(x) / np.float32(8.0)
    beta = _sigmoid(y)
    return PrefillInputs("gdn", dtype, _store(q, dtype), _store(k, dtype), _store(v, dtype),
                         _store(g, dtype), _store(beta, dtype), w.astype(np.float32),
                         np.full((H,), b_lam, dtype=np.float32))


def structured_inputs(rule: str, B: int, H: int, T: int, d: int, seed: int,
                      dtype: str = "bf16", rank: int = 4, needle_every: int = 64,
                      b_lam: float = 0.0) -> PrefillInputs:
    """Keys concentrated on a low-rank 'haystack' subspace plus isolated needles.

    A synthetic stand-in for the pages' premise that the wanted key sits off the
    high-variance subspace of the key covariance (10100.com write-up, section
    "记忆体检"): haystack keys are normalize(A z + 0.1 eps) with A in
    R^{d x rank} per head, and every ``needle_every``-th key is a random unit
    vector.  b_lambda = 0 gives lambda near 0.5, so the cleaning term is a
    sizeable part of the output.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, d), dtype=np.float32)
    A = rng.standard_normal((B, H, d, rank), dtype=np.float32)
    z = rng.standard_normal((B, H, T, rank), dtype=np.float32)
    eps = rng.standard_normal((B, H, T, d), dtype=np.float32)
    needles = rng.standard_normal((B, H, T, d), dtype=np.float32)
    k = np.einsum("bhdr,bhtr->bhtd", A, z).astype(np.float32) + np.float32(0.1) * eps
    if needle_every > 0:
        k[:, :, needle_every - 1::needle_every] = needles[:, :, needle_every - 1::needle_every]
    k = _unit_rows(k)
    v = rng.standard_normal((B, H, T, d), dtype=np.float32)
    w = None
    if rule == "gla":
        x = rng.standard_normal((B, H, T, d), dtype=np.float32)
        g = _logsigmoid(x) / np.float32(16.0)
        beta = None
    elif rule == "gdn":
        x = rng.standard_normal((B, H, T), dtype=np.float32)
        y = rng.standard_normal((B, H, T), dtype=np.float32)
        g = -_softplus(x) / np.float32(8.0)
        beta = _store(_sigmoid(y), dtype)
    else:
        raise ValueError(rule)
    w = rng.standard_normal((H, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    return PrefillInputs(rule, dtype, _store(q, dtype), _store(k, dtype), _store(v, dtype),
                         _store(g, dtype), beta, w.astype(np.float32),
                         np.full((H,), b_lam, dtype=np.float32))


def subspace_keys(B: int, H: int, T: int, d: int, seed: int, dtype: str = "bf16", rank: int = 16,
                  needle_every: int = 64):
    """Keys for the key-covariance subspace diagnostic, and their needle mask.

    Haystack keys are normalize(Q diag(s) z + 0.1 eps) with Q a random d x rank orthonormal
    basis per head and s spread evenly over [2, 1], so the key covariance has ``rank``
    distinct leading eigenvalues well above the rest; every ``needle_every``-th key is a
    random unit vector (a needle, mostly off that subspace).  A stand-in for the retrieval
    prompts of the 10100.com write-up's section "记忆体检".  Returns (k [B, H, T, d] stored
    in dtype, as fp32; needle [B, H, T] bool)."""
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((B, H, d, rank))
    Q, _ = np.linalg.qr(G)
    s = np.linspace(2.0, 1.0, rank)
    z = rng.standard_normal((B, H, T, rank))
    eps = rng.standard_normal((B, H, T, d))
    k = np.einsum("bhdr,bhtr->bhtd", Q * s, z) + 0.1 * eps
    needle = np.zeros((B, H, T), dtype=bool)
    if needle_every > 0:
        needle[:, :, needle_every - 1::needle_every] = True
        k[needle] = rng.standard_normal((int(needle.sum()), d))
    k = _unit_rows(k.astype(np.float32))
    return _store(k, dtype), needle


def decode_tokens(rule: str, N: int, H: int, d: int, seed: int, dtype: str = "bf16"):
    """One new token per (sequence, head): dict of [N, H, d] / [N, H] fp32 arrays."""
    x = gla_inputs(N, H, 1, d, seed, dtype) if rule == "gla" else gdn_inputs(N, H, 1, d, seed, dtype)
    out = dict(q=x.q[:, :, 0], k=x.k[:, :, 0], v=x.v[:, :, 0], g=x.g[:, :, 0],
               beta=None if x.beta is None else x.beta[:, :, 0],
               w_lam=x.w_lam, b_lam=x.b_lam)
    return out


# The measured workloads.  Index 0 is the small fp32 case the oracle finishes in
# seconds; 1 is the headline prefill; 4 is the decode step.
WORKLOADS = {
    0: dict(name="ccq-gla-fwd-f32-B1H2T256d64", rule="gla", dtype="f32", B=1, H=2, T=256, d=64, seed=1000),
    1: dict(name="ccq-gla-fwd-bf16-B4H16T4096d128", rule="gla", dtype="bf16", B=4, H=16, T=4096, d=128, seed=1001),
    2: dict(name="ccq-gdn-fwd-bf16-B4H16T4096d128", rule="gdn", dtype="bf16", B=4, H=16, T=4096, d=128, seed=1002),
    3: dict(name="ccq-gla-fwd-bf16-B1H16T20480d128", rule="gla", dtype="bf16", B=1, H=16, T=20480, d=128, seed=1003),
    4: dict(name="ccq-gla-decode-N256H16d128-n8192", rule="gla", dtype="bf16", N=256, H=16, T=8192, d=128,
            seed=1004, token_seed=2004),
}


def workload_inputs(i: int) -> PrefillInputs:
    """Prefill inputs of workload 0-3 (workload 4's prefix is built on the device)."""
    w = WORKLOADS[i]
    if i == 4:
        raise ValueError("the decode workload's 8K-token prefix is generated on the device")
    gen = gla_inputs if w["rule"] == "gla" else gdn_inputs
    return gen(w["B"], w["H"], w["T"], w["d"], w["seed"], w["dtype"])

"""What the GPU's CCQ-delta check can detect (CPU only; the slip is planted in a private copy of the
oracle, never in the real module).

The GPU check compares o(b_lambda) - o(b_lambda = -inf), both stored in bf16, with the oracle's
exact delta on keys whose haystack lies on a low-rank subspace (the cleaning removes a large part
of the read: the pages' premise that the wanted key sits off the high-variance subspace, 10100.com
write-up, section "记忆体检"; the cleaning itself, gist.science summary §2 "机制").  Here the same
comparison runs on the oracle's own outputs rounded to bf16, once exact and once with the cleaning
term scaled by (1 + eps): the exact outputs must stay well inside each bound (the bf16 storage of
the outputs is most of the error the GPU check sees), and a cleaning term a few percent off must
fail it.
"""

import os
import types

import numpy as np
import pytest

import oracle
from curvature_conditioned_query_amd.inputs import bf16_round, structured_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ANCHOR = "q_clean = qt - lam[..., None] * np.matmul(Sigma, qt[..., None])[..., 0]"

# the GPU test's bounds, by haystack rank (tests/test_gpu_contract.py)
BOUND = {4: 3e-2, 2: 2e-2}
# (rank, the smallest planted eps that the bound must reject)
CASES = [(4, 0.05), (2, 0.03)]


def _scaled_cleaning_oracle():
    src = open(os.path.join(ROOT, "oracle", "ccq.py")).read()
    assert src.count(ANCHOR) == 1
    mod = types.ModuleType("oracle_scaled_cleaning")
    exec(compile(src.replace(ANCHOR, ANCHOR.replace("lam[..., None]", "(1.0 + EPS) * lam[..., None]")),
                 "<scaled cleaning>", "exec"), mod.__dict__)
    return mod


def _bf16(a):
    return bf16_round(np.asarray(a, np.float32)).astype(np.float64)


@pytest.mark.parametrize("rule", ["gla", "gdn"])
@pytest.mark.parametrize("rank,eps_reject", CASES)
def test_delta_bound_rejects_a_scaled_cleaning_term(rule, rank, eps_reject):
    x = structured_inputs(rule, 1, 1, 1024, 128, 3140 + rank, "bf16", rank=rank, b_lam=3.0)
    o_ref, _ = oracle.ccq_recurrent(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule)
    b = x.b_lam.copy()
    x.b_lam[:] = -np.inf
    o0_ref, _ = oracle.ccq_recurrent(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule)
    x.b_lam[:] = b
    dref = o_ref - o0_ref
    assert np.abs(dref).max() / np.abs(o_ref).max() > (0.25 if rank == 4 else 0.6)
    m = _scaled_cleaning_oracle()
    errs = {}
    for eps in (0.0, eps_reject):
        m.EPS = eps
        ob, _ = m.ccq_recurrent(x.q, x.k, x.v, x.g, x.beta, x.w_lam, x.b_lam, rule)
        errs[eps] = oracle.normwise_error(_bf16(ob) - _bf16(o0_ref), dref)
    print(f"{rule} rank {rank}: delta err of bf16 outputs {errs[0.0]:.3e}, with the cleaning x (1 + {eps_reject}) "
          f"{errs[eps_reject]:.3e}, bound {BOUND[rank]:.0e}")
    assert errs[0.0] < 0.7 * BOUND[rank]
    assert errs[eps_reject] > BOUND[rank]

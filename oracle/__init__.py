"""CPU fp64 oracle for the Curvature-Conditioned Query read step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only the tests, the graft smoke check and the benchmark's CPU
baseline leg do.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or constant generators); the only thing both sides share is the
seeded input generator, which holds none of the method's arithmetic.

Sources, cited by page title and section:

* "技术摘要：不要阅读一切：一种基于曲率条件的线性注意力查询" (gist.science summary
  of arXiv 2606.01294), §2 "理论推导" (log-partition and its second-order
  expansion, running mean and second moment), §2 "机制" (cleaned query, gate,
  extra d_k x d_k matrix and d_k vector per head), §2 "集成" (write rule
  unchanged, o_t = S_t q_t^clean).
* "EMNLP 2026 最佳论文｜Linear attention 的大海捞针，能否从“读”这一步改进？"
  (10100.com write-up), section "方法解析" (Hessian = unweighted key covariance,
  one scalar gate per token and head, unit keys give eig in [1-lambda, 1]) and
  section "代价与边界" (the covariance is undecayed).
* The two write rules the pages name but do not print are the standard ones:
  GLA, S_t = S_{t-1} diag(alpha_t) + v_t k_t^T with alpha per key channel, and
  Gated DeltaNet, S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.

* The gradients of the recurrence (``grad.py``): the forward step once more in plain
  PyTorch fp64, differentiated by torch.autograd, pinned to finite differences.
* The key-covariance subspace diagnostic (``subspace.py``) follows the 10100.com
  write-up's section "记忆体检" (Δμ: needle vs distractor alignment with the top-16
  eigen-subspace of the key covariance).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force, library routines and hand-derived fixtures
(``tests/golden``).  No function is left "parity unpinned".
"""

from .ccq import (  # noqa: F401
    Carry,
    ccq_chunked,
    ccq_decode_step,
    ccq_recurrent,
    gla_closed_form_carry,
    key_covariance,
    normwise_error,
    pack_upper,
    sigmoid,
    unit_keys,
    unpack_upper,
)
from .subspace import covariance_from_sums, delta_mu, subspace_alignment, top_eigen  # noqa: F401
from .grad import ccq_sequence_backward, ccq_step_backward, ccq_step_torch  # noqa: F401

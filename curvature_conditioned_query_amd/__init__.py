"""MI355X-native Curvature-Conditioned Query (CCQ) read step.

The compute path is the C-ABI library ``libccq.so`` (hand-written HIP for
gfx950), declared in ``include/ccq.h``.  ``ccq`` below is a thin ctypes binding
that marshals torch tensors into that ABI; every step of the method runs in the
library's kernels.  Importing this package does not load the library; the first
call does, and raises if it is missing.
"""

from .binding import (  # noqa: F401
    CCQ_RULE_GLA,
    CCQ_RULE_GDN,
    CcqError,
    ccq_decode_step,
    ccq_fwd_chunked,
    ccq_fwd_chunked_noalloc,
    ccq_fwd_workspace_bytes,
    ccq_key_subspace,
    ccq_bwd_chunked,
    ccq_chunk_carry_bytes,
    ccq_step_backward,
    new_chunk_carry,
    library_path,
    load_library,
)

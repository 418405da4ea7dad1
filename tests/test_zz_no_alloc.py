"""ccq_fwd_chunked_noalloc against ccq_fwd_chunked, through the C ABI on the GPU.

The no-allocation entry point takes its workspace from a device array inside the library; every
call on a device shares it and leaves its contents behind.  Two calls in a row (the second on a
smaller input, so it reads a shorter stretch of an array the first call filled) must each give
exactly what ccq_fwd_chunked gives on the same inputs with the same segment split, and the
default split must stay within the bf16 bar of it.
"""

import numpy as np
import pytest

from curvature_conditioned_query_amd.inputs import gdn_inputs, gla_inputs
from oracle import Carry, normwise_error

from gpu_util import down, up_carry, upload_inputs

pytestmark = pytest.mark.gpu


def _run(fn, x, segments, carry=None, alias=False, packed=False):
    import torch
    d = upload_inputs(x)
    B, H, T, dk, dv = x.shape
    cin = None if carry is None else up_carry(carry)[0]
    if alias and cin is not None:
        cout = cin
    else:
        cout = (torch.empty((B, H, dv, dk), device="cuda"),
                torch.empty((B, H, dk * (dk + 1) // 2) if packed else (B, H, dk, dk), device="cuda"),
                torch.empty((B, H, dk), device="cuda"), torch.empty((B, H), dtype=torch.int64, device="cuda"))
    if packed and cin is not None:
        raise ValueError("packed carry in is not used here")
    o = fn(x.rule, d["q"], d["k"], d["v"], d["g"], d["beta"], d["w"], d["b"], carry_in=cin, carry_out=cout,
           segments=segments, packed_cov=packed)
    torch.cuda.synchronize()
    return down(o), tuple(down(t) for t in cout)


def _both(x, segments, **kw):
    from curvature_conditioned_query_amd import ccq_fwd_chunked, ccq_fwd_chunked_noalloc
    ref = _run(ccq_fwd_chunked, x, segments, **kw)
    got = _run(ccq_fwd_chunked_noalloc, x, segments, **kw)
    return got, ref


def _same(got, ref, tag):
    (o, c), (o_r, c_r) = got, ref
    print(f"{tag}: o max |diff| {np.max(np.abs(o - o_r)):.3e}", flush=True)
    assert np.array_equal(o, o_r), tag
    for a, b in zip(c, c_r):
        assert np.array_equal(a, b), tag


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_noalloc_two_calls_match_the_workspace_entry_point(gpu_lib, rule):
    gen = gla_inputs if rule == "gla" else gdn_inputs
    # first call: the benchmark shape's chain count with 4 segments (34-50 MB of the 64 MiB array)
    big = gen(4, 16, 1024, 128, 7101, "bf16")
    _same(*_both(big, 4), tag=f"{rule} B4 H16 T1024 seg 4")
    # second call, smaller, right after it: 6 chains x 3 segments
    small = gen(2, 3, 330, 128, 7102, "bf16")
    _same(*_both(small, 3), tag=f"{rule} B2 H3 T330 seg 3")


@pytest.mark.parametrize("rule", ["gla", "gdn"])
def test_noalloc_default_segments_and_aliased_carry(gpu_lib, rule):
    """Default split (the library's own, shortened only if its workspace would not fit) within the
    bf16 bar of ccq_fwd_chunked's; then a carry in aliased by the carry out with several segments,
    which goes through the copy of the carry in the array holds."""
    from oracle import ccq_recurrent
    gen = gla_inputs if rule == "gla" else gdn_inputs
    x = gen(1, 4, 700, 128, 7103, "bf16")
    (o, c), (o_r, c_r) = _both(x, 0)
    e = normwise_error(o, o_r)
    print(f"{rule} default segments: o err vs ccq_fwd_chunked {e:.3e}", flush=True)
    assert e <= 2e-2
    assert np.array_equal(c[3], c_r[3])
    x0 = gen(1, 4, 90, 128, 7104, "f32")
    _, pre = ccq_recurrent(x0.q, x0.k, x0.v, x0.g, x0.beta, x0.w_lam, x0.b_lam, rule)
    (_, (S, C, m, n)) = up_carry(pre)
    carry = Carry(S, C, m, n)
    _same(*_both(x, 5, carry=carry, alias=True), tag=f"{rule} aliased carry seg 5")

"""The benchmark's algorithmic work counts and its one-GPU contract (CPU only).

The roofline figures bench.py reports divide these counts by measured times, so each is pinned
here to a count derived separately from what the kernels must read, write and multiply.
"""

import os
import subprocess
import sys

import bench

L = 64  # chunk length


def test_prefill_flops_per_token_head():
    """GLA chunk form, every product counted as full tiles: Q K^T, tril(P) K, the intra attention
    matrix and its product with V are L x L x d (4 of them); Q C0, Qc S0^T, K^T K and the S update
    are L x d x d (4 of them): 2 (4 L^2 d + 4 L d^2) per chunk of L tokens."""
    d = 128
    per_chunk = 2 * (4 * L * L * d + 4 * L * d * d)
    flops, _ = bench.prefill_work(1, 1, L, d, 2)
    assert flops == per_chunk
    flops, _ = bench.prefill_work(4, 16, 4096, d, 2)
    assert flops == 4 * 16 * 64 * per_chunk == 51_539_607_552


def test_prefill_bytes_headline():
    """q, k, v, log alpha read and o written once in bf16, and the fp32 carry out (S, C, ksum)
    with the int64 count per chain."""
    B, H, T, d = 4, 16, 4096, 128
    tokens = B * H * T * (4 * d * 2 + d * 2)
    carry = B * H * (2 * d * d * 4 + d * 4 + 8)
    _, nbytes = bench.prefill_work(B, H, T, d, 2)
    assert nbytes == tokens + carry == 343_966_208


def test_main_kernel_bytes_with_segments():
    """The main kernel also reads the carry-in slots (S, C, ksum in fp32) of segments 1..P-1."""
    B, H, T, d, P = 4, 16, 4096, 128, 4
    expect = B * H * T * 5 * d * 2 + B * H * (P - 1) * (2 * d * d + d) * 4 + B * H * (2 * d * d * 4 + d * 4 + 8)
    assert bench.main_kernel_bytes(B, H, T, d, 2, P) == expect == 369_230_336
    # one segment: no slots
    assert bench.main_kernel_bytes(B, H, T, d, 2, 1) == 369_230_336 - 3 * 64 * (2 * d * d + d) * 4


def test_prefill_roofline_uses_the_algorithmic_bytes():
    """frac divides the pass's algorithmic bytes (343,966,208 at the headline shape), not the main
    kernel's own reads of the segment carry-ins, by the main kernel's launch duration."""
    res = dict(shape=(4, 16, 4096, 128, 128), spec=dict(rule="gla", name="w"), segments=4,
               phase_ms=dict(summary=0.05, scan=0.01, main=0.1))
    flops, nbytes = bench.prefill_work(4, 16, 4096, 128, 2)
    roof = bench.prefill_roofline(res, flops, nbytes, 2, "0" * 64)
    assert roof["algorithmic_bytes_per_launch"] == 343_966_208
    assert roof["achieved"] == round(343_966_208 / 1e-4 / 1e9, 1)
    assert roof["frac"] == round(343_966_208 / 1e-4 / 8e12, 4)
    assert roof["kernel_bytes_with_segment_carries"] == 369_230_336
    assert roof["traffic"] is None and roof["mfma"]["counter_busy_frac"] is None


def test_gdn_prefill_counts():
    d = 128
    flops, nbytes = bench.prefill_work(1, 1, L, d, 2, "gdn")
    # the CCQ part as for GLA (Q K^T, tril(P) K, Q C0, K^T K) plus K K^T, U, W, Qc K^T, M Delta on
    # L x L tiles, and W S0^T, Qc S0^T, the S update on d x d: 2 (7 L^2 d + 5 L d^2) per chunk
    assert flops == 2 * (7 * L * L * d + 5 * L * d * d)
    assert nbytes == L * (3 * d * 2 + 2 * 2 + d * 2) + (2 * d * d * 4 + d * 4 + 8)


def test_decode_bytes_per_head_step():
    d = 128
    full = 4 * d * d * 4 + 2 * d * 4 + 2 * 8 + 4 * d * 2 + d * 2
    assert bench.decode_bytes_per_head(d, 2) == full == 264_464
    packed = 2 * (d * d + d * (d + 1) // 2) * 4 + 2 * d * 4 + 2 * 8 + 4 * d * 2 + d * 2
    assert bench.decode_bytes_per_head(d, 2, packed_cov=True) == packed == 199_440


def test_step_backward_bytes_per_head_step():
    """S, C, dS, dC read and dS, dC written (fp32 d x d); token and w read; ksum, n, d_o, dksum in
    and dksum out; dq, dk, dv, dlog alpha, dw written (fp32 d) and db."""
    d = 128
    expect = 6 * d * d * 4 + 4 * d * 2 + d * 4 + (d * 4 + 8) + d * 4 + 2 * d * 4 + 5 * d * 4 + 4
    assert bench.step_backward_bytes_per_head(d, 2) == expect == 399_372


def test_bwd_chunk_work():
    d = 128
    fa, fb, ba = bench.bwd_chunk_work(d, 2)
    assert fa == 2 * (5 * L * d * d + 8 * L * L * d) == 18_874_368
    assert fb == 2 * (3 * L * d * d + 4 * L * L * d) == 10_485_760
    reads = 5 * L * d * 2 + 2 * d * d * 2 + 2 * d * 4
    writes = 4 * L * d * 4 + 2 * d * d * 2 + 4 * d * 4
    assert ba == reads + writes == 347_136


def test_gdn_bwd_chunk_work():
    """Gated DeltaNet chunked backward per chunk: pass A has 7 L x d x d products (Q C_c, dR C_c,
    dR^T Q, K S_c^T, dO^T (gamma Qc), Z'^T (beta gamma K), dO S_c) and 14 L x L x d ones; pass B 6
    and 11.  Pass A reads q, k, v, d_o (bf16), log alpha and beta, S_c and C_c (bf16), m_c and w;
    writes qc, dq and the partial dk (fp32), the 64 x 64 inverse, R_c and dG_c (bf16), the tails."""
    d = 128
    fa, fb, ba = bench.gdn_bwd_chunk_work(d, 2)
    assert fa == 2 * (7 * L * d * d + 14 * L * L * d) == 29_360_128
    assert fb == 2 * (6 * L * d * d + 11 * L * L * d) == 24_117_248
    reads = 4 * L * d * 2 + 2 * L * 2 + 2 * d * d * 2 + 2 * d * 4
    writes = 3 * L * d * 4 + L * L * 2 + 2 * d * d * 2 + 4 * d * 4
    assert ba == reads + writes


def test_eigen_flops():
    """d = 128, r = 16, 10 multisection rounds per eigenvalue: 4/3 d^3 for the tridiagonal form,
    4 points x 4 flops x d per round, 36 d per vector of inverse iteration, 2 x 120 pairs x 4d of
    Gram-Schmidt, 4 r sum_{m=2}^{d-1} m of back-transformation."""
    d, r = 128, 16
    back = 4 * r * (d * (d - 1) // 2 - 1)
    assert bench.eigen_flops(d, r, 10 * d) == 2_796_202 + 2_621_440 + 73_728 + 122_880 + back
    assert bench.eigen_flops(d, r, 0) == bench.eigen_flops(d, r, 10 * d) - 2_621_440


def test_more_than_one_gpu_is_refused():
    """The benchmark measures one GPU; asking for more exits with status 2 and says so."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)

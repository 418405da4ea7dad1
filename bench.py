#!/usr/bin/env python3
"""Benchmark of the CCQ read step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1] [--no-cpu] [--no-decode]

A step is one chunked-prefill pass of a CCQ-GLA layer over one batch of synthetic
input (B=4, H=16, T=4096, d_k=d_v=128, bf16 q/k/v/log-decay, fp32 carry out), with
the inputs resident in HBM.  ``value`` is prefill tokens/s (B*T per second).  The
same run times the decode step (256 sequences x 16 heads, d=128, a carry pre-filled
from an 8K-token prefix) and reports its HBM bandwidth, times the same GLA layer on 5x
longer sequences (B=1, H=16, T=20480: per-token time against T=4096), and times the fp64
CPU oracle on a bounded sample of the prefill workload.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA, TFLOP/s
CHUNK = 64
MALL_FLUSH_BYTES = 512 << 20  # written between the flushed passes: twice the MI355X's 256 MB MALL


# ------------------------------------------------------------------ algorithmic work
def prefill_work(B, H, T, d, elem_bytes, rule="gla"):
    """Algorithmic flops and HBM bytes of one prefill pass.

    flops per (token, head): GLA 8 d^2 + 8 L d (full 16x16 MFMA tiles of the L=64 chunk
    form: Q K^T, Q C0, tril(P) K, Qc S0^T, the intra attention matrix and its product
    with V, K^T K and the S update); Gated DeltaNet 10 d^2 + 14 L d (the CCQ part as for GLA,
    plus K K^T, U = T diag(beta) V, W = T diag(beta gamma) K, Qc K^T and its product with Delta
    on L x L tiles, W S0^T, Qc S0^T and the S update on d x d; the L^3/3 solve is not counted).
    bytes: q, k, v, log decay read once and o written once, plus the fp32 carry out
    (S, C, ksum, n) per chain."""
    th = B * H * T
    if rule == "gla":
        flop_th = 8 * d * d + 8 * CHUNK * d
        in_bytes_th = 4 * d * elem_bytes
    else:
        flop_th = 10 * d * d + 14 * CHUNK * d
        in_bytes_th = 3 * d * elem_bytes + 2 * elem_bytes
    bytes_th = in_bytes_th + d * elem_bytes
    carry = 2 * d * d * 4 + d * 4 + 8
    return th * flop_th, th * bytes_th + B * H * carry


def main_kernel_bytes(B, H, T, d, elem_bytes, segments, rule="gla"):
    """Algorithmic HBM bytes of one launch of the main prefill kernel: q, k, v and the gates
    (GLA: log decay per key channel; GDN: log alpha and beta per token) read and o written
    once, the carry-in of every segment after the first read from the workspace (S, C, ksum
    in fp32), and the final carry (S, C, ksum, n) written."""
    chains = B * H
    per_th = (5 * d if rule == "gla" else 4 * d + 2) * elem_bytes
    tokens = B * H * T * per_th
    slot_in = (2 * d * d + d) * 4
    carry_out = 2 * d * d * 4 + d * 4 + 8
    return tokens + chains * (max(segments, 1) - 1) * slot_in + chains * carry_out


def decode_bytes_per_head(d, elem_bytes, packed_cov=False):
    """S (fp32 d x d) and C (fp32 d x d, or its d (d + 1) / 2 packed upper triangle) read and
    written, ksum read and written, n read and written, one token (q, k, v, log alpha) read,
    o written."""
    c_floats = d * (d + 1) // 2 if packed_cov else d * d
    return 2 * (d * d + c_floats) * 4 + 2 * d * 4 + 2 * 8 + 4 * d * elem_bytes + d * elem_bytes


def file_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def library_sha():
    """Hash of every library source, header and compile flag (the one the profiles/ records store)."""
    from curvature_conditioned_query_amd.build import library_sha256
    return library_sha256()


def _profile_record(name, lib_sha):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("library_sha256") != lib_sha:
        return None
    return rec


def measured_traffic(name, lib_sha):
    """HBM bytes per launch from a committed rocprofv3 --pmc record, if it was taken on the library
    as it is now (every source, header and flag), else None."""
    rec = _profile_record(name, lib_sha)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def measured_mfma(name, lib_sha):
    """Counter-based MFMA-pipe utilisation from a committed record, if taken on the current library."""
    rec = _profile_record(name, lib_sha)
    return None if rec is None else rec.get("mfma_busy_frac")


# ------------------------------------------------------------------ GPU legs
def to_dev(x, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype).contiguous()


def time_prefill(wl, steps, warmup, keep_outputs=False, flushed=100):
    import torch
    from curvature_conditioned_query_amd import ccq_fwd_chunked, load_library
    from curvature_conditioned_query_amd.inputs import WORKLOADS, workload_inputs
    load_library()
    spec = WORKLOADS[wl]
    x = workload_inputs(wl)
    tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    B, H, T, dk, dv = x.shape
    q, k, v, g = (to_dev(a, tdt) for a in (x.q, x.k, x.v, x.g))
    beta = None if x.beta is None else to_dev(x.beta, tdt)
    w = torch.from_numpy(x.w_lam).cuda()
    b = torch.from_numpy(x.b_lam).cuda()
    o = torch.empty((B, H, T, dv), dtype=tdt, device="cuda")
    cout = (torch.empty((B, H, dv, dk), device="cuda"), torch.empty((B, H, dk, dk), device="cuda"),
            torch.empty((B, H, dk), device="cuda"), torch.empty((B, H), dtype=torch.int64, device="cuda"))
    from curvature_conditioned_query_amd.binding import make_fwd_params, ccq_fwd_workspace_bytes
    p = make_fwd_params(x.rule, q, k, v, g, beta, w, b, o, None, cout)
    ws_bytes = ccq_fwd_workspace_bytes(p)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    del x

    hip = HipEvents(4 * steps)

    def step(i=None):
        pe = None if i is None else hip.slice(4 * i, 4)
        ccq_fwd_chunked(spec["rule"], q, k, v, g, beta, w, b, o=o, carry_out=cout, workspace=ws,
                        phase_events=pe)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # the throughput: K back-to-back passes with nothing else on the stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = e0.elapsed_time(e1)
    # per-kernel launch durations: K more passes with the events the library records on its
    # stream around its kernels (each record adds a few microseconds between the kernels,
    # so these passes are not the ones the throughput comes from)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    phases = {name: float(np.mean([hip.elapsed_ms(4 * i + a, 4 * i + a + 1) for i in range(steps)]))
              for a, name in enumerate(("summary", "scan", "main"))}
    hip.destroy()
    # `flushed` more passes, each after an untimed 512 MB write that evicts the MALL (so every pass
    # reads its inputs from HBM), each timed alone with events on the launch stream; the median
    # is reported beside the back-to-back rate
    flushed_ms = []
    if flushed > 0:
        buf = torch.empty(MALL_FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(flushed)]
        for i, (a0, a1) in enumerate(evs):
            buf.fill_(float(i))
            a0.record(stream)
            step()
            a1.record(stream)
        torch.cuda.synchronize()
        flushed_ms = [a0.elapsed_time(a1) for a0, a1 in evs]
        del buf
    outputs = None
    if keep_outputs:  # the timed passes' o and final carry (every pass writes the same values)
        outputs = {"o": o.float().cpu().numpy(), "S": cout[0].cpu().numpy(), "C": cout[1].cpu().numpy(),
                   "ksum": cout[2].cpu().numpy(), "n": cout[3].cpu().numpy()}
    # segments the library resolved: its workspace holds one fp32 slot per (chain, segment)
    # when there is more than one segment (GLA: S, C, ksum, log decay; GDN: S, C, ksum, M)
    slot = (2 * dk * dk + 2 * dk) * 4 if spec["rule"] == "gla" else (3 * dk * dk + dk) * 4
    segs = int(p.segments) if p.segments else (ws_bytes // (B * H * slot) or 1)
    return dict(spec=spec, shape=(B, H, T, dk, dv), total_ms=total_ms, per_ms=per, wall_s=t_wall,
                dtype=spec["dtype"], workspace_bytes=ws_bytes, segments=segs, phase_ms=phases, outputs=outputs,
                flushed_ms=flushed_ms)


def prefill_roofline(res, flops, nbytes, elem, lib_sha):
    """Roofline of a prefill pass's dominant kernel, the main kernel (one launch per pass).

    achieved = the pass's algorithmic bytes (q, k, v and the gates read once, o written once, the
    final carry written: the work of the whole layer, none of it intermediate) over the main
    kernel's average launch duration; frac = achieved / 8 TB/s.  The main kernel's own bytes
    (those plus the segment carry-ins it reads from the workspace, an intermediate of the segment
    split) are reported beside it, as is the method's flop rate over the same duration and the
    counter-based MFMA-pipe utilisation of the kernel when a record of it matches the library."""
    B, H, T, dk, _ = res["shape"]
    spec = res["spec"]
    main_ms = res["phase_ms"]["main"]
    mfma_peak = BF16_PEAK_TFLOPS if elem == 2 else FP32_PEAK_TFLOPS
    k_gbs = nbytes / (main_ms * 1e-3) / 1e9
    k_tflops = flops / (main_ms * 1e-3) / 1e12
    # the GLA prefill at d = 128 with 16-bit inputs (keys not normalised in the kernel, as here)
    # runs the pipelined main kernel, every other GLA case the single-role one
    if spec["rule"] == "gla":
        kname = "gla_pipe_kernel" if (dk == 128 and elem == 2) else "gla_main_kernel"
    else:
        kname = "gdn_main_kernel"
    return dict(bound="hbm", achieved=round(k_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(k_gbs / HBM_PEAK_GBS, 4),
                traffic=measured_traffic(f"traffic_{spec['name']}.json", lib_sha),
                kernel=f"{kname}<{dk},{'bf16' if elem == 2 else 'f32'}>", avg_launch_ms=round(main_ms, 4),
                algorithmic_bytes_per_launch=nbytes, algorithmic_flops_per_launch=flops,
                kernel_bytes_with_segment_carries=main_kernel_bytes(B, H, T, dk, elem, res["segments"] or 1,
                                                                    spec["rule"]),
                mfma=dict(achieved=round(k_tflops, 1), peak=mfma_peak, unit="TFLOP/s",
                          frac=round(k_tflops / mfma_peak, 4),
                          counter_busy_frac=measured_mfma(f"mfma_{spec['name']}.json", lib_sha)),
                pass_ms={k: round(v, 4) for k, v in res["phase_ms"].items()})


def flushed_summary(res, tokens):
    """Median (and spread) of the MALL-flushed passes of a prefill leg."""
    f = res["flushed_ms"]
    if not f:
        return None
    med = float(np.median(f))
    return dict(passes=len(f), median_ms=round(med, 4), min_ms=round(float(np.min(f)), 4),
                max_ms=round(float(np.max(f)), 4), tokens_per_s=round(tokens / (med * 1e-3), 1),
                flush_bytes=MALL_FLUSH_BYTES)


class HipEvents:
    """Plain hipEvent_t handles from the HIP runtime torch has loaded (same soname, so the
    same runtime instance the kernels are launched through)."""

    def __init__(self, n):
        import ctypes
        self._ct = ctypes
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev[i] = h

    def slice(self, i, n):
        ct = self._ct
        return ct.cast(ct.byref(self.ev, i * ct.sizeof(ct.c_void_p)), ct.POINTER(ct.c_void_p))

    def elapsed_ms(self, i, j):
        ms = self._ct.c_float()
        if self.rt.hipEventElapsedTime(self._ct.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self):
        for h in self.ev:
            self.rt.hipEventDestroy(h)


# (sequence, head) pairs of the decode workload whose prefix, carry and first step are kept on the
# host for the oracle check in the CPU leg
DECODE_SAMPLES = ((0, 0), (131, 7), (255, 15))


def time_decode(steps, warmup, seqs_per_batch=32, packed_cov=False, keep_samples=False):
    """Decode workload: 256 sequences x 16 heads, d=128, carry from an 8192-token prefix
    built by the prefill kernel on device-generated seeded inputs.  packed_cov: the statistic
    C is kept as its packed upper triangle (prefill writes it so, decode updates it so).
    keep_samples: host copies, for the sampled heads, of the prefix, of the carry the prefill
    built from it, and of the first decode step's token, output and carry after it (that step
    runs before the warm-up; the timed steps follow from its state)."""
    import torch
    from curvature_conditioned_query_amd import ccq_decode_step, ccq_fwd_chunked
    from curvature_conditioned_query_amd.inputs import WORKLOADS
    spec = WORKLOADS[4]
    N, H, T, d = spec["N"], spec["H"], spec["T"], spec["d"]
    bf = torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(spec["seed"])
    S = torch.empty((N, H, d, d), device="cuda")
    C = torch.empty((N, H, d * (d + 1) // 2) if packed_cov else (N, H, d, d), device="cuda")
    m = torch.empty((N, H, d), device="cuda")
    n = torch.empty((N, H), dtype=torch.int64, device="cuda")
    w = (torch.randn((H, d), generator=gen, device="cuda") / np.sqrt(d)).float().contiguous()
    b = torch.full((H,), -2.0, device="cuda")
    samples = {}
    for s0 in range(0, N, seqs_per_batch):
        nb = min(seqs_per_batch, N - s0)
        shp = (nb, H, T, d)
        qq = torch.randn(shp, generator=gen, device="cuda").to(bf)
        kk = torch.randn(shp, generator=gen, device="cuda")
        kk = (kk / kk.norm(dim=-1, keepdim=True)).to(bf)
        vv = torch.randn(shp, generator=gen, device="cuda").to(bf)
        gg = (torch.nn.functional.logsigmoid(torch.randn(shp, generator=gen, device="cuda")) / 16).to(bf)
        if keep_samples:
            for (sq, hh) in DECODE_SAMPLES:
                if s0 <= sq < s0 + nb:
                    samples[(sq, hh)] = {name: t[sq - s0, hh].float().cpu().numpy()
                                         for name, t in (("q", qq), ("k", kk), ("v", vv), ("g", gg))}
        ccq_fwd_chunked("gla", qq, kk, vv, gg, None, w, b,
                        carry_out=(S[s0:s0 + nb], C[s0:s0 + nb], m[s0:s0 + nb], n[s0:s0 + nb]),
                        packed_cov=packed_cov)
        del qq, kk, vv, gg
    torch.cuda.synchronize()
    gen.manual_seed(spec["token_seed"])
    tq = torch.randn((N, H, d), generator=gen, device="cuda").to(bf)
    tk = torch.randn((N, H, d), generator=gen, device="cuda")
    tk = (tk / tk.norm(dim=-1, keepdim=True)).to(bf)
    tv = torch.randn((N, H, d), generator=gen, device="cuda").to(bf)
    tg = (torch.nn.functional.logsigmoid(torch.randn((N, H, d), generator=gen, device="cuda")) / 16).to(bf)
    o = torch.empty((N, H, d), dtype=bf, device="cuda")

    def step():
        ccq_decode_step("gla", tq, tk, tv, tg, None, w, b, S, C, m, n, o=o, packed_cov=packed_cov)

    def carry_of(sq, hh):
        return tuple(t[sq, hh].cpu().numpy().copy() for t in (S, C, m, n))

    if keep_samples:
        for (sq, hh), rec in samples.items():
            rec["carry"] = carry_of(sq, hh)
            rec["token"] = {name: t[sq, hh].float().cpu().numpy() for name, t in
                            (("q", tq), ("k", tk), ("v", tv), ("g", tg))}
        step()
        torch.cuda.synchronize()
        for (sq, hh), rec in samples.items():
            rec["o"] = o[sq, hh].float().cpu().numpy()
            rec["carry_after"] = carry_of(sq, hh)
        wh, bh = w.cpu().numpy(), b.cpu().numpy()
        for (sq, hh), rec in samples.items():
            rec["w"], rec["b"] = wh[hh:hh + 1], bh[hh:hh + 1]
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = N * H * decode_bytes_per_head(d, 2, packed_cov)
    name = spec["name"].replace("decode-", "decode-packed-") if packed_cov else spec["name"]
    del S, C, m, n
    return dict(spec=spec, name=name, ms_per_step=ms, bytes_per_step=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
                tokens_per_s=N / (ms * 1e-3), samples=samples, packed_cov=packed_cov)


def time_subspace(calls, warmup, r=16):
    """Key-covariance subspace diagnostic on B=4, H=16, T=4096, d=128 bf16 keys with 16 leading
    directions and a needle every 64 tokens; the statistics come from a GLA prefill of those
    keys (the carry), the call computes eigenvalues, the top-16 basis, every key's alignment
    and Δμ per head."""
    import torch
    from curvature_conditioned_query_amd import ccq_fwd_chunked, ccq_key_subspace
    from curvature_conditioned_query_amd.inputs import subspace_keys
    B, H, T, d = 4, 16, 4096, 128
    k_np, needle_np = subspace_keys(B, H, T, d, 1005, "bf16")
    bf = torch.bfloat16
    k = torch.from_numpy(k_np).cuda().to(bf)
    needle = torch.from_numpy(needle_np).cuda()
    gen = torch.Generator(device="cuda").manual_seed(1005)
    q = torch.randn((B, H, T, d), generator=gen, device="cuda").to(bf)
    v = torch.randn((B, H, T, d), generator=gen, device="cuda").to(bf)
    g = (torch.nn.functional.logsigmoid(torch.randn((B, H, T, d), generator=gen, device="cuda")) / 16).to(bf)
    w = (torch.randn((H, d), generator=gen, device="cuda") / np.sqrt(d)).contiguous()
    b = torch.full((H,), -2.0, device="cuda")
    S = torch.empty((B, H, d, d), device="cuda")
    C = torch.empty((B, H, d * (d + 1) // 2), device="cuda")
    m = torch.empty((B, H, d), device="cuda")
    n = torch.empty((B, H), dtype=torch.int64, device="cuda")
    ccq_fwd_chunked("gla", q, k, v, g, None, w, b, carry_out=(S, C, m, n), packed_cov=True)
    for _ in range(warmup):
        out = ccq_key_subspace(C, m, n, k, r=r, needle=needle, packed_cov=True)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        out = ccq_key_subspace(C, m, n, k, r=r, needle=needle, packed_cov=True)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    dmu = out[3].float().cpu().numpy()
    iters = torch.empty((B, H), dtype=torch.int32, device="cuda")
    ccq_key_subspace(C, m, n, k, r=r, needle=needle, packed_cov=True, iters=iters)
    torch.cuda.synchronize()
    it = iters.cpu().numpy()
    return dict(name=f"ccq-key-subspace-B{B}H{H}T{T}d{d}-r{r}", ms=ms, heads=B * H, tokens=B * T,
                delta_mu_mean=float(np.nanmean(dmu)), iters=it,
                flops=sum(eigen_flops(d, r, int(x)) for x in it.ravel()))


def step_backward_bytes_per_head(d, elem_bytes):
    """Algorithmic HBM bytes of one backward step per (sequence, head): S, C and the adjoints dS,
    dC (fp32 d x d) read, dS and dC written back; the token (q, k, v, log alpha) and w_lambda
    read; ksum, n, d_o read, dksum read and written; dq, dk, dv, dlog_alpha, dw_lambda (fp32 d)
    and db_lambda written."""
    return 6 * d * d * 4 + 4 * d * elem_bytes + d * 4 + d * 4 + 8 + d * 4 + 2 * d * 4 + 5 * d * 4 + 4


def time_step_backward(steps, warmup, rule="gla"):
    """Backward of one recurrence step over the decode workload's shape (256 sequences x 16 heads,
    d = 128, bf16 token, fp32 state and adjoints), K times in a row (the adjoints are updated in
    place, as when walking a sequence backwards)."""
    import torch
    from curvature_conditioned_query_amd import ccq_step_backward
    N, H, d = 256, 16, 128
    gen = torch.Generator(device="cuda").manual_seed(1006)
    bf = torch.bfloat16
    K = torch.randn((N, H, 32, d), generator=gen, device="cuda")
    K = K / K.norm(dim=-1, keepdim=True)
    C = 64 * (K.transpose(-1, -2).contiguous() @ K)
    C = ((C + C.transpose(-1, -2)) / 2).contiguous()
    m = (64 * K.sum(dim=2)).contiguous()
    del K
    n = torch.full((N, H), 2048, dtype=torch.int64, device="cuda")
    S = (torch.randn((N, H, d, d), generator=gen, device="cuda") / np.sqrt(d)).contiguous()
    dS = torch.zeros((N, H, d, d), device="cuda")
    dC = torch.zeros((N, H, d, d), device="cuda")
    dm = torch.zeros((N, H, d), device="cuda")
    do = torch.randn((N, H, d), generator=gen, device="cuda")
    q = torch.randn((N, H, d), generator=gen, device="cuda").to(bf)
    k = torch.randn((N, H, d), generator=gen, device="cuda")
    k = (k / k.norm(dim=-1, keepdim=True)).to(bf)
    v = torch.randn((N, H, d), generator=gen, device="cuda").to(bf)
    if rule == "gla":
        g = (torch.nn.functional.logsigmoid(torch.randn((N, H, d), generator=gen, device="cuda")) / 16).to(bf)
        beta = None
    else:
        g = (-torch.nn.functional.softplus(torch.randn((N, H), generator=gen, device="cuda")) / 8).to(bf)
        beta = torch.sigmoid(torch.randn((N, H), generator=gen, device="cuda")).to(bf)
    w = (torch.randn((H, d), generator=gen, device="cuda") / np.sqrt(d)).contiguous()
    b = torch.full((H,), -2.0, device="cuda")

    def step():
        ccq_step_backward(rule, q, k, v, g, beta, w, b, S, C, m, n, do, dS, dC, dm)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = N * H * step_backward_bytes_per_head(d, 2)
    return dict(name=f"ccq-{rule}-step-backward-N{N}H{H}d{d}", ms=ms, bytes=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9)


def bwd_chunk_work(d, elem_bytes, L=CHUNK):
    """Per 64-token chunk of the chunked backward: algorithmic flops of pass A and pass B (every
    matrix product of the chunk algebra counted dense, 2 m n k; pass A: Q K^T, Q C_c, tril(P) K,
    dO V^T, dO^T (qc e^B), dO S_c, tril(D) (k e^-B), dR K^T, dR C_c, tril(M) K, P^T dR, M^T Q,
    dR^T Q; pass B: (qc e^B)(k e^-B)^T, dO V^T, A^T dO, D^T (qc e^B), (k e^-B) dS^T, V dS,
    K (G + G^T)) and pass A's algorithmic HBM bytes (q, k, v, log alpha, d_o read; S_c, C_c,
    ksum_c, w read; qc, qc * dqc, dq and the partial dk written, fp32; R_c, dG_c and the chunk
    sums written)."""
    flops_a = 2 * (5 * L * d * d + 8 * L * L * d)
    flops_b = 2 * (3 * L * d * d + 4 * L * L * d)
    # the chunk carry (S_c, C_c) and the adjoint matrices (R_c, dG_c) are stored in the input dtype
    bytes_a = (5 * L * d * elem_bytes + 2 * d * d * elem_bytes + 2 * d * 4 + 4 * L * d * 4
               + 2 * d * d * elem_bytes + 4 * d * 4)
    return flops_a, flops_b, bytes_a


def gdn_bwd_chunk_work(d, elem_bytes, L=CHUNK):
    """Per 64-token chunk of the Gated DeltaNet chunked backward: algorithmic flops of pass A and pass
    B (every matrix product counted dense, 2 m n k; pass A: the read's Q K^T, Q C_c, tril(P) K,
    dR C_c, dR K^T, M2 K, P^T dR, M2^T Q, dR^T Q, and the rule's K K^T, K S_c^T, T X, Qc K^T, M^T dO,
    T^T Z, dO Delta^T, dO^T (gamma Qc), Z'^T (beta gamma K), dO S_c, (dM Gam) K; pass B: K (G + G^T),
    K S_c^T, T X, Qc K^T, dO Delta^T, M^T dO, K dS_L^T, T^T dDelta, dX Delta^T, K K^T, (dM Gam)^T Qc,
    W_A K, W_A^T K, dX S_c, Delta dS_L, Qc S_c^T) and pass A's algorithmic HBM bytes (q, k, v, d_o,
    log alpha, beta read; S_c, C_c, m_c, w read; qc, dq and the partial dk written, fp32; the
    64 x 64 inverse, R_c and dG_c written in the input dtype; the chunk sums written)."""
    flops_a = 2 * (7 * L * d * d + 14 * L * L * d)
    flops_b = 2 * (6 * L * d * d + 11 * L * L * d)
    bytes_a = (4 * L * d * elem_bytes + 2 * L * elem_bytes + 2 * d * d * elem_bytes + 2 * d * 4
               + 3 * L * d * 4 + L * L * elem_bytes + 2 * d * d * elem_bytes + 4 * d * 4)
    return flops_a, flops_b, bytes_a


def time_bwd_chunked(steps, warmup, rule="gla"):
    """Chunked backward over a prefill benchmark's inputs (B = 4, H = 16, T = 4096, d = 128, bf16,
    zero carry; GLA on the headline prefill's inputs, Gated DeltaNet on its own prefill's) with a
    seeded bf16 output gradient; the carry-out adjoint is zero."""
    import torch
    from curvature_conditioned_query_amd import ccq_bwd_chunked, load_library
    from curvature_conditioned_query_amd.inputs import WORKLOADS, workload_inputs
    load_library()
    wl = 1 if rule == "gla" else 2
    x = workload_inputs(wl)
    B, H, T, dk, dv = x.shape
    bf = torch.bfloat16
    q, k, v, g = (to_dev(a, bf) for a in (x.q, x.k, x.v, x.g))
    beta = None if x.beta is None else to_dev(x.beta, bf)
    w = torch.from_numpy(x.w_lam).cuda()
    b = torch.from_numpy(x.b_lam).cuda()
    del x
    gen = torch.Generator(device="cuda").manual_seed(1007)
    do = torch.randn((B, H, T, dv), generator=gen, device="cuda").to(bf)
    out = ccq_bwd_chunked(rule, q, k, v, g, w, b, do, beta=beta)  # allocates the outputs
    ws = torch.empty(int(_ws_bytes_bwd(B, H, T, dk, rule)), dtype=torch.uint8, device="cuda")
    hip = HipEvents(5 * steps)

    def step(i=None):
        pe = None if i is None else hip.slice(5 * i, 5)
        return ccq_bwd_chunked(rule, q, k, v, g, w, b, do, workspace=ws, phase_events=pe, beta=beta)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    phases = {name: float(np.mean([hip.elapsed_ms(5 * i + a, 5 * i + a + 1) for i in range(steps)]))
              for a, name in enumerate(("carries", "pass_a", "scan", "pass_b"))}
    hip.destroy()
    # training with the forward's chunk carries: the prefill writing them (against the plain
    # prefill), then the backward reading them instead of recomputing them
    from curvature_conditioned_query_amd import ccq_fwd_chunked, new_chunk_carry
    from curvature_conditioned_query_amd.binding import ccq_fwd_workspace_bytes, make_fwd_params
    o = torch.empty_like(do)
    fws_n = ccq_fwd_workspace_bytes(make_fwd_params(rule, q, k, v, g, beta, w, b, o))
    fws = torch.empty(max(fws_n, 1), dtype=torch.uint8, device="cuda") if fws_n else None
    cc = new_chunk_carry(q)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(steps):
            fn()
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / steps

    fwd_ms = timed(lambda: ccq_fwd_chunked(rule, q, k, v, g, beta, w, b, o=o, workspace=fws))
    fwd_cc_ms = timed(lambda: ccq_fwd_chunked(rule, q, k, v, g, beta, w, b, o=o, workspace=fws, chunk_carry=cc))
    bwd_cc_ms = timed(lambda: ccq_bwd_chunked(rule, q, k, v, g, w, b, do, workspace=ws, beta=beta, chunk_carry=cc))
    del out, cc
    return dict(name=f"ccq-{rule}-bwd-chunked-B{B}H{H}T{T}d{dk}-bf16", shape=(B, H, T, dk, dv), ms=ms,
                phase_ms=phases, chunks=B * H * ((T + CHUNK - 1) // CHUNK), rule=rule,
                with_chunk_carries=dict(forward_ms=fwd_ms, forward_writing_carries_ms=fwd_cc_ms,
                                        backward_reading_carries_ms=bwd_cc_ms))


def _ws_bytes_bwd(B, H, T, d, rule="gla"):
    import ctypes
    from curvature_conditioned_query_amd.binding import BwdParams, load_library
    p = BwdParams()
    p.rule, p.dtype, p.B, p.H, p.T, p.d_k, p.d_v, p.chunk = (0 if rule == "gla" else 1), 1, B, H, T, d, d, CHUNK
    names = ["q", "k", "v", "log_alpha", "w_lambda", "b_lambda", "d_o", "dq", "dk", "dv", "dlog_alpha", "dw_lambda",
             "db_lambda"] + ([] if rule == "gla" else ["beta", "dbeta"])
    for n in names:
        setattr(p, n, 1 << 20)  # aligned placeholders: only the size query reads this struct
    return load_library().ccq_bwd_workspace_bytes(ctypes.byref(p))


def bwd_chunked_entry(cres, lib_sha):
    """The JSON entry of a chunked-backward leg: time per pass, per-pass times from the library's
    events, and pass A's roofline (algorithmic bytes and flops per chunk x chunks, over its event-timed
    launch duration; pass B's flop rate beside it)."""
    cB, cH, cT, cd, _ = cres["shape"]
    fa, fb, ba = bwd_chunk_work(cd, 2) if cres["rule"] == "gla" else gdn_bwd_chunk_work(cd, 2)
    pa = cres["phase_ms"]["pass_a"]
    a_tf = fa * cres["chunks"] / (pa * 1e-3) / 1e12
    a_gbs = ba * cres["chunks"] / (pa * 1e-3) / 1e9
    pb = cres["phase_ms"]["pass_b"]
    b_tf = fb * cres["chunks"] / (pb * 1e-3) / 1e12
    kern = "bwd_chunk_a_kernel" if cres["rule"] == "gla" else "gdn_bwd_a_kernel"
    print(f"# {cres['name']}: {cres['ms']:.3f} ms/pass, {cB * cT / (cres['ms'] * 1e-3):.4g} tokens/s; "
          "passes (ms) " + ", ".join(f"{k} {v:.4f}" for k, v in cres["phase_ms"].items())
          + f"; pass A {a_gbs:.1f} GB/s alg, {a_tf:.1f} TFLOP/s, pass B {b_tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    wc = cres["with_chunk_carries"]
    print(f"#   with the forward's chunk carries: forward {wc['forward_ms']:.3f} -> {wc['forward_writing_carries_ms']:.3f} "
          f"ms, backward {wc['backward_reading_carries_ms']:.3f} ms (forward + backward {wc['forward_ms'] + cres['ms']:.3f} "
          f"-> {wc['forward_writing_carries_ms'] + wc['backward_reading_carries_ms']:.3f} ms)", file=sys.stderr, flush=True)
    return {
        "with_chunk_carries": {k: round(v, 4) for k, v in wc.items()},
        "workload": cres["name"], "ms_per_step": round(cres["ms"], 4),
        "tokens_per_s": round(cB * cT / (cres["ms"] * 1e-3), 1),
        "pass_ms": {k: round(v, 4) for k, v in cres["phase_ms"].items()},
        "roofline": dict(bound="hbm", achieved=round(a_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(a_gbs / HBM_PEAK_GBS, 4),
                         traffic=measured_traffic(f"traffic_{cres['name']}.json", lib_sha),
                         kernel=f"{kern}<{cd},bf16>", avg_launch_ms=round(pa, 4),
                         algorithmic_flops_per_launch=fa * cres["chunks"],
                         algorithmic_bytes_per_launch=ba * cres["chunks"],
                         intensity_flop_per_byte=round(fa / ba, 1),
                         ridge_flop_per_byte=round(BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9), 1),
                         mfma=dict(achieved=round(a_tf, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                                   frac=round(a_tf / BF16_PEAK_TFLOPS, 4)),
                         pass_b=dict(achieved=round(b_tf, 1), unit="TFLOP/s", frac=round(b_tf / BF16_PEAK_TFLOPS, 4))),
    }


EIG_THREADS = 512  # the eigen kernel's workgroup: 512 / d lanes per eigenvalue in the multisection


def eigen_flops(d, r, rounds):
    """Algorithmic fp32 flops of one head's eigen-decomposition (d x d, top-r vectors) with
    ``rounds`` multisection rounds summed over its eigenvalues: the Householder tridiagonalisation
    (4/3 d^3, the standard count), the Sturm counts (4 flops per term, 512 / d points per round),
    three inverse-iteration solves per vector (12 flops per row), two Gram-Schmidt passes (a dot
    and an update, 4d flops per pair) and the back-transformation (4 flops per entry of each
    reflector, per vector)."""
    tri = 4 * d ** 3 // 3
    sturm = rounds * (EIG_THREADS // d) * 4 * d
    inv = 3 * 12 * d * r
    mgs = 2 * (r * (r - 1) // 2) * 4 * d
    back = sum(4 * (d - k - 1) for k in range(d - 2)) * r
    return tri + sturm + inv + mgs + back


# ------------------------------------------------------------------ CPU oracle leg
def _oracle_slab(args):
    """Times the oracle on one chain; with the GPU's output for that chain (o, and the final
    carry when the whole chain was run) also returns the normwise errors against it."""
    import oracle
    q, k, v, g, beta, w, b, rule, gpu = args
    t = time.perf_counter()
    o_ref, c_ref = oracle.ccq_recurrent(q, k, v, g, beta, w, b, rule)
    dt = time.perf_counter() - t
    if gpu is None:
        return dt, None
    errs = {"o": oracle.normwise_error(gpu["o"], o_ref)}
    if "S" in gpu:
        errs["S"] = oracle.normwise_error(gpu["S"], c_ref.S)
        errs["C"] = oracle.normwise_error(gpu["C"], c_ref.C)
        errs["ksum"] = oracle.normwise_error(gpu["ksum"][..., None], c_ref.m[..., None])
        errs["n_exact"] = bool(np.array_equal(gpu["n"], c_ref.n))
    return dt, errs


def cpu_baseline(wl, tokens, max_workers, gpu_out=None):
    """The fp64 recurrent oracle, as it is, on every (b, h) chain of the workload but only the
    first `tokens` tokens of each; one chain slab per worker process, one BLAS thread each.
    With gpu_out (host copies of the timed passes' o and final carry) each worker also compares
    the GPU's result for its chain with the oracle's."""
    import concurrent.futures as cf
    from curvature_conditioned_query_amd.inputs import workload_inputs
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    x = workload_inputs(wl)
    B, H, T, dk, dv = x.shape
    tokens = min(tokens, T)
    jobs = []
    for bb in range(B):
        for hh in range(H):
            sl = x.slab(bb, hh, 0, tokens)
            gpu = None
            if gpu_out is not None:
                gpu = {"o": gpu_out["o"][bb:bb + 1, hh:hh + 1, :tokens]}
                if tokens == T:
                    for name in ("S", "C", "ksum", "n"):
                        gpu[name] = gpu_out[name][bb:bb + 1, hh:hh + 1]
            jobs.append((sl.q, sl.k, sl.v, sl.g, sl.beta, sl.w_lam, sl.b_lam, x.rule, gpu))
    workers = max(1, min(max_workers, len(jobs)))
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(_oracle_slab, jobs))
    wall = time.perf_counter() - t0
    cpu_s = sum(r[0] for r in res)
    errs = [r[1] for r in res if r[1] is not None]
    parity = None
    if errs:
        parity = {key: (all(e[key] for e in errs) if key == "n_exact" else max(e[key] for e in errs))
                  for key in errs[0]}
        parity.update(chains=len(errs), tokens=tokens)
    return dict(value=B * tokens / wall, unit="tokens/s", cores=workers, kind="oracle",
                sample=f"all {B * H} (b,h) chains of the workload, first {tokens} of {T} tokens each; "
                       f"fp64 per-token recurrence; {workers} worker processes; {cpu_s:.1f} CPU-s, {wall:.1f} s wall",
                wall_s=wall, cpu_s=cpu_s, parity=parity)


def decode_parity(samples, packed_cov, cache):
    """The oracle on the sampled heads of the decode leg: the carry after the 8192-token prefix
    (against the carry the prefill kernel built) and one decode step from the GPU's own carry
    (against the GPU step's output and carry after it).  Normwise errors, max over the samples;
    `cache` keeps the prefix runs, which both decode legs share."""
    import oracle
    errs = {}

    def upd(key, e):
        errs[key] = max(errs.get(key, 0.0), e)

    n_exact = True
    for key, rec in samples.items():
        if key not in cache:
            pre = {name: rec[name][None, None] for name in ("q", "k", "v", "g")}
            cache[key] = oracle.ccq_recurrent(pre["q"], pre["k"], pre["v"], pre["g"], None, rec["w"], rec["b"],
                                              "gla")[1]
        ref = cache[key]
        d = rec["carry"][0].shape[-1]

        def full_c(c):
            return oracle.unpack_upper(c, d) if packed_cov else c

        S, C, m, n = rec["carry"]
        upd("prefix_S", oracle.normwise_error(S[None, None], ref.S))
        upd("prefix_C", oracle.normwise_error(full_c(C)[None, None], ref.C))
        upd("prefix_ksum", oracle.normwise_error(m[None, None, :, None], ref.m[..., None]))
        n_exact &= bool(np.array_equal(np.asarray(n).reshape(1, 1), ref.n))
        gc = oracle.Carry(S[None, None].astype(np.float64), full_c(C)[None, None].astype(np.float64),
                          m[None, None].astype(np.float64), np.asarray(n, np.int64).reshape(1, 1))
        tok = {name: rec["token"][name][None, None] for name in ("q", "k", "v", "g")}
        o_ref, c_ref = oracle.ccq_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], None, rec["w"], rec["b"], "gla",
                                              gc)
        S1, C1, m1, n1 = rec["carry_after"]
        upd("step_o", oracle.normwise_error(rec["o"][None, None, :, None], o_ref[..., None]))
        upd("step_S", oracle.normwise_error(S1[None, None], c_ref.S))
        upd("step_C", oracle.normwise_error(full_c(C1)[None, None], c_ref.C))
        upd("step_ksum", oracle.normwise_error(m1[None, None, :, None], c_ref.m[..., None]))
        n_exact &= bool(np.array_equal(np.asarray(n1).reshape(1, 1), c_ref.n))
    tol = 2e-2
    out = {k: round(v, 8) for k, v in errs.items()}
    out.update(n_exact=n_exact, samples=[list(k) for k in samples], tolerance=tol,
               against="fp64 per-token recurrence (oracle)",
               **{"pass": bool(n_exact and all(v <= tol for v in errs.values()))})
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------ main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 3])
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gdn", action="store_true", help="skip the Gated DeltaNet prefill leg")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context (T=20480) prefill leg")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill leg (profiling the decode kernel alone)")
    ap.add_argument("--no-subspace", action="store_true", help="skip the key-subspace diagnostic leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the step-backward leg")
    ap.add_argument("--backward-only", action="store_true", help="run the step-backward leg alone")
    ap.add_argument("--subspace-only", action="store_true", help="run the key-subspace diagnostic leg alone")
    ap.add_argument("--no-bwd-chunked", action="store_true", help="skip the chunked-backward leg")
    ap.add_argument("--bwd-chunked-only", action="store_true", help="run the chunked-backward leg alone")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain streaming kernel over MIB MiB (torch.neg, 3 times), the reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # streams n*4 bytes in and n*4 bytes out
        torch.cuda.synchronize()
        del src, dst
    if args.backward_only:
        for rule in ("gla", "gdn"):
            bres = time_step_backward(args.decode_steps, 3, rule)
            print(f"# {bres['name']}: {bres['ms'] * 1e3:.1f} us/step, {bres['gbs']:.1f} GB/s", file=sys.stderr,
                  flush=True)
        return 0
    if args.bwd_chunked_only:
        lib_sha = library_sha()
        for rule in ("gla", "gdn"):
            bwd_chunked_entry(time_bwd_chunked(args.steps, args.warmup, rule=rule), lib_sha)  # prints its lines
        return 0
    if args.subspace_only:
        sres = time_subspace(5, 1)
        print(f"# {sres['name']}: {sres['ms']:.3f} ms/call, multisection rounds per head {sres['iters'].min()}..{sres['iters'].max()}, "
              f"{sres['flops'] / (sres['ms'] * 1e-3) / 1e12:.3f} TFLOP/s", file=sys.stderr, flush=True)
        return 0
    if args.no_prefill:
        for packed in (False, True):
            dres = time_decode(args.decode_steps, 3, packed_cov=packed)
            print(f"# {dres['name']}: {dres['ms_per_step']*1e3:.1f} us/step, {dres['gbs']:.1f} GB/s",
                  file=sys.stderr, flush=True)
        return 0
    res = time_prefill(args.workload, args.steps, args.warmup, keep_outputs=not args.no_cpu)
    B, H, T, dk, dv = res["shape"]
    spec = res["spec"]
    elem = 2 if res["dtype"] == "bf16" else 4
    flops, nbytes = prefill_work(B, H, T, dk, elem, spec["rule"])
    ms = res["total_ms"] / args.steps
    tok_s = B * T / (ms * 1e-3)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    mfma_peak = BF16_PEAK_TFLOPS if res["dtype"] == "bf16" else FP32_PEAK_TFLOPS
    intensity = flops / nbytes
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    lib_sha = library_sha()
    roof = prefill_roofline(res, flops, nbytes, elem, lib_sha)
    roof.update(whole_pass=dict(bytes=nbytes, gbs=round(gbs, 1), tflops=round(tflops, 1),
                                hbm_frac=round(gbs / HBM_PEAK_GBS, 4)),
                bound_by_intensity="hbm" if intensity < ridge else "mfma",
                flushed=flushed_summary(res, B * T))
    out = {
        "metric": "CCQ-GLA prefill tokens/s (H16,dk128,T4K) + MFMA util; decode HBM GB/s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic (seeded normal q, v; unit-normalised keys; logsigmoid(x)/16 log decay; bf16)",
        "config": {"workload": spec["name"], "rule": spec["rule"], "B": B, "H": H, "T": T, "d_k": dk,
                   "d_v": dv, "chunk": CHUNK, "segments": res["segments"], "carry": "fp32"},
        "roofline": roof,
    }
    print(f"# prefill {spec['name']}: {ms:.3f} ms/step, {tok_s:.4g} tokens/s, {gbs:.1f} GB/s alg, "
          f"{tflops:.1f} TFLOP/s alg; kernels (ms) " +
          ", ".join(f"{k} {v:.4f}" for k, v in res["phase_ms"].items()), file=sys.stderr, flush=True)
    if not args.no_long and args.workload == 1:
        # the pages' systems claim is that CCQ's cost does not grow with sequence length: the same
        # layer on 5x longer sequences (B=1, H=16, T=20480), per-token time against the line above
        lres = time_prefill(3, args.steps, args.warmup, flushed=0)
        lB, lH, lT = lres["shape"][:3]
        l_ms = lres["total_ms"] / args.steps
        ns_tok = l_ms * 1e6 / (lB * lH * lT)
        ns_tok_1 = ms * 1e6 / (B * H * T)
        out["long_context"] = {
            "workload": lres["spec"]["name"], "ms_per_step": round(l_ms, 4),
            "tokens_per_s": round(lB * lT / (l_ms * 1e-3), 1), "segments": lres["segments"],
            "pass_ms": {k: round(v, 4) for k, v in lres["phase_ms"].items()},
            "ns_per_token_head": round(ns_tok, 4), "ns_per_token_head_T4096": round(ns_tok_1, 4),
            "ratio_to_T4096": round(ns_tok / ns_tok_1, 3)}
        print(f"# prefill {lres['spec']['name']}: {l_ms:.3f} ms/step, {ns_tok:.4f} ns per (token, head) "
              f"against {ns_tok_1:.4f} at T=4096", file=sys.stderr, flush=True)
    if not args.no_gdn:
        gres = time_prefill(2, args.steps, args.warmup)
        gB, gH, gT, gd, _ = gres["shape"]
        g_ms = gres["total_ms"] / args.steps
        g_flops, g_bytes = prefill_work(gB, gH, gT, gd, 2, "gdn")
        g_main = gres["phase_ms"]["main"]
        groof = prefill_roofline(gres, g_flops, g_bytes, 2, lib_sha)
        groof["flushed"] = flushed_summary(gres, gB * gT)
        g_gbs, g_tf = groof["achieved"], groof["mfma"]["achieved"]
        out["gdn"] = {
            "workload": gres["spec"]["name"], "ms_per_step": round(g_ms, 4),
            "tokens_per_s": round(gB * gT / (g_ms * 1e-3), 1), "segments": gres["segments"],
            "pass_ms": {k: round(v, 4) for k, v in gres["phase_ms"].items()},
            "roofline": groof,
        }
        print(f"# prefill {gres['spec']['name']}: {g_ms:.3f} ms/step, {gB * gT / (g_ms * 1e-3):.4g} tokens/s, "
              f"main kernel {g_main:.4f} ms, {g_gbs:.1f} GB/s alg, {g_tf:.1f} TFLOP/s alg",
              file=sys.stderr, flush=True)
    decode_samples = {}
    if not args.no_decode:
        for key, packed in (("decode", False), ("decode_packed", True)):
            dres = time_decode(args.decode_steps, 3, packed_cov=packed, keep_samples=not args.no_cpu)
            decode_samples[key] = (dres["samples"], packed)
            out[key] = {
                "workload": dres["name"], "ms_per_step": round(dres["ms_per_step"], 4),
                "tokens_per_s": round(dres["tokens_per_s"], 1), "packed_cov": packed,
                "roofline": dict(bound="hbm", achieved=round(dres["gbs"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                                 frac=round(dres["gbs"] / HBM_PEAK_GBS, 4),
                                 traffic=measured_traffic(f"traffic_{dres['name']}.json", lib_sha)),
                "algorithmic_bytes_per_step": dres["bytes_per_step"],
            }
            print(f"# {dres['name']}: {dres['ms_per_step']*1e3:.1f} us/step, {dres['gbs']:.1f} GB/s",
                  file=sys.stderr, flush=True)
    if not args.no_backward:
        out["step_backward"] = {}
        for rule in ("gla", "gdn"):
            bres = time_step_backward(args.decode_steps, 3, rule)
            out["step_backward"][rule] = {
                "workload": bres["name"], "ms_per_step": round(bres["ms"], 4),
                "roofline": dict(bound="hbm", achieved=round(bres["gbs"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                                 frac=round(bres["gbs"] / HBM_PEAK_GBS, 4),
                                 traffic=measured_traffic(f"traffic_{bres['name']}.json", lib_sha)),
                "algorithmic_bytes_per_step": bres["bytes"]}
            print(f"# {bres['name']}: {bres['ms'] * 1e3:.1f} us/step, {bres['gbs']:.1f} GB/s", file=sys.stderr,
                  flush=True)
    if not args.no_bwd_chunked:
        cres = time_bwd_chunked(args.steps, args.warmup)
        out["bwd_chunked"] = bwd_chunked_entry(cres, lib_sha)
        gcres = time_bwd_chunked(args.steps, args.warmup, rule="gdn")
        out["bwd_chunked_gdn"] = bwd_chunked_entry(gcres, lib_sha)
    if not args.no_subspace:
        sres = time_subspace(5, 1)
        s_tf = sres["flops"] / (sres["ms"] * 1e-3) / 1e12
        out["subspace"] = {"workload": sres["name"], "ms_per_call": round(sres["ms"], 4),
                           "heads_per_s": round(sres["heads"] / (sres["ms"] * 1e-3), 1),
                           "delta_mu_mean": round(sres["delta_mu_mean"], 4),
                           "multisection_rounds": {"min": int(sres["iters"].min()), "max": int(sres["iters"].max()),
                                                   "mean": round(float(sres["iters"].mean()), 2)},
                           "roofline": dict(bound="alu", achieved=round(s_tf, 3), peak=FP32_PEAK_TFLOPS,
                                            unit="TFLOP/s", frac=round(s_tf / FP32_PEAK_TFLOPS, 5),
                                            traffic=None, kernel="subspace_eigen_kernel<128> (with the "
                                            "alignment and delta kernels in the timed call)",
                                            algorithmic_flops_per_call=sres["flops"])}
        print(f"# {sres['name']}: {sres['ms']:.3f} ms/call (eigen-decomposition of {sres['heads']} heads, "
              f"alignment of {sres['tokens']} tokens x 16 heads), mean delta-mu {sres['delta_mu_mean']:+.4f}",
              file=sys.stderr, flush=True)
    if not args.no_cpu:
        try:
            ncpu = len(os.sched_getaffinity(0))
        except AttributeError:
            ncpu = os.cpu_count() or 1
        cb = cpu_baseline(args.workload, args.cpu_tokens, min(ncpu, 16), gpu_out=res["outputs"])
        cb["cpu_model"] = cpu_model()
        out["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample", "cpu_model")}
        print(f"# cpu oracle: {cb['value']:.4g} tokens/s on {cb['cores']} cores ({cb['wall_s']:.1f} s wall)",
              file=sys.stderr, flush=True)
        cache = {}
        for key, (smp, packed) in decode_samples.items():
            if smp:
                out[key]["parity"] = decode_parity(smp, packed, cache)
                print(f"# {key} parity on {len(smp)} sampled heads: " + ", ".join(
                    f"{k} {v:.3e}" for k, v in out[key]["parity"].items() if isinstance(v, float)),
                      file=sys.stderr, flush=True)
        if cb["parity"] is not None:
            # the timed passes' own output against the oracle, normwise per (b, h) chain (max over
            # chains), at the tolerance the inputs' precision sets
            tol = 2e-2 if res["dtype"] == "bf16" else 1e-4
            par = dict(cb["parity"], tolerance=tol, against="fp64 per-token recurrence (oracle)")
            par["pass"] = bool(all(v <= tol for k, v in par.items() if k in ("o", "S", "C", "ksum"))
                               and par.get("n_exact", True))
            out["parity"] = {k: (round(v, 8) if isinstance(v, float) else v) for k, v in par.items()}
            print(f"# parity of the timed passes' output: " + ", ".join(
                f"{k} {v:.3e}" for k, v in cb["parity"].items() if isinstance(v, float)), file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

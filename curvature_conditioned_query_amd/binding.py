"""ctypes binding of ``libccq.so`` (the C ABI in ``include/ccq.h``).

Argument marshalling only: torch tensors are checked for device, dtype and
contiguity and handed to the library as raw device pointers together with the
caller's current HIP stream.  No step of the method runs here, and there is no
fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

CCQ_RULE_GLA = 0
CCQ_RULE_GDN = 1
CCQ_DTYPE_F32 = 0
CCQ_DTYPE_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

# Every symbol include/ccq.h declares (kept in one place for the export test).
EXPORTED_SYMBOLS = (
    "ccq_fwd_chunked",
    "ccq_fwd_chunked_noalloc",
    "ccq_fwd_workspace_bytes",
    "ccq_decode_step",
    "ccq_key_subspace",
    "ccq_step_backward",
    "ccq_bwd_chunked",
    "ccq_bwd_workspace_bytes",
    "ccq_chunk_carry_bytes",
    "ccq_status_string",
    "ccq_abi_version",
)


class CcqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({_status_string(status)})")


class FwdParams(ctypes.Structure):
    """Mirror of ``ccq_fwd_params``."""

    _fields_ = [
        ("rule", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("chunk", ctypes.c_int32), ("segments", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("log_alpha", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("w_lambda", ctypes.c_void_p), ("b_lambda", ctypes.c_void_p),
        ("S0", ctypes.c_void_p), ("C0", ctypes.c_void_p), ("ksum0", ctypes.c_void_p),
        ("n0", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("S_out", ctypes.c_void_p), ("C_out", ctypes.c_void_p), ("ksum_out", ctypes.c_void_p),
        ("n_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("phase_events", ctypes.c_void_p),
        ("flags", ctypes.c_int32),
        ("chunk_carry", ctypes.c_void_p),
    ]


class BwdParams(ctypes.Structure):
    """Mirror of ``ccq_bwd_params``."""

    _fields_ = [
        ("rule", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p),
        ("w_lambda", ctypes.c_void_p), ("b_lambda", ctypes.c_void_p),
        ("S0", ctypes.c_void_p), ("C0", ctypes.c_void_p), ("ksum0", ctypes.c_void_p), ("n0", ctypes.c_void_p),
        ("d_o", ctypes.c_void_p),
        ("dS_T", ctypes.c_void_p), ("dC_T", ctypes.c_void_p), ("dksum_T", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p), ("dlog_alpha", ctypes.c_void_p),
        ("dw_lambda", ctypes.c_void_p), ("db_lambda", ctypes.c_void_p),
        ("dS0", ctypes.c_void_p), ("dC0", ctypes.c_void_p), ("dksum0", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("phase_events", ctypes.c_void_p),
        ("flags", ctypes.c_int32),
        ("beta", ctypes.c_void_p), ("dbeta", ctypes.c_void_p),
        ("chunk_carry", ctypes.c_void_p),
    ]


def library_path() -> str:
    return os.environ.get("CCQ_LIBRARY", os.path.join(_HERE, "libccq.so"))


def load_library():
    """Load libccq.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m curvature_conditioned_query_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.ccq_fwd_chunked.argtypes = [ctypes.POINTER(FwdParams), vp]
    lib.ccq_fwd_chunked.restype = ctypes.c_int
    lib.ccq_fwd_chunked_noalloc.argtypes = [ctypes.POINTER(FwdParams), vp]
    lib.ccq_fwd_chunked_noalloc.restype = ctypes.c_int
    lib.ccq_fwd_workspace_bytes.argtypes = [ctypes.POINTER(FwdParams)]
    lib.ccq_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ccq_decode_step.argtypes = [i32, i32, i32, i32, i32, i32] + [vp] * 12 + [i32, vp]
    lib.ccq_decode_step.restype = ctypes.c_int
    lib.ccq_key_subspace.argtypes = [i32] * 6 + [vp] * 10 + [i32, vp]
    lib.ccq_key_subspace.restype = ctypes.c_int
    lib.ccq_step_backward.argtypes = [i32] * 6 + [vp] * 22 + [i32, vp]
    lib.ccq_step_backward.restype = ctypes.c_int
    lib.ccq_bwd_chunked.argtypes = [ctypes.POINTER(BwdParams), vp]
    lib.ccq_bwd_chunked.restype = ctypes.c_int
    lib.ccq_bwd_workspace_bytes.argtypes = [ctypes.POINTER(BwdParams)]
    lib.ccq_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ccq_chunk_carry_bytes.argtypes = [i32] * 5
    lib.ccq_chunk_carry_bytes.restype = ctypes.c_size_t
    lib.ccq_status_string.argtypes = [i32]
    lib.ccq_status_string.restype = ctypes.c_char_p
    lib.ccq_abi_version.argtypes = []
    lib.ccq_abi_version.restype = i32
    _LIB = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().ccq_status_string(status).decode()
    except Exception:  # pragma: no cover - only used for messages
        return "?"


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return CCQ_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return CCQ_DTYPE_BF16
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check_dev(name, t, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _rule_code(rule) -> int:
    if rule in ("gla", CCQ_RULE_GLA):
        return CCQ_RULE_GLA
    if rule in ("gdn", CCQ_RULE_GDN):
        return CCQ_RULE_GDN
    raise ValueError(f"unknown rule {rule!r}")


FLAG_NORMALIZE_KEYS = 1  # CCQ_FLAG_NORMALIZE_KEYS
FLAG_PACKED_COV = 2  # CCQ_FLAG_PACKED_COV


def _flags(normalize_keys: bool, packed_cov: bool) -> int:
    return (FLAG_NORMALIZE_KEYS if normalize_keys else 0) | (FLAG_PACKED_COV if packed_cov else 0)


def _check_numel(name, t, n):
    if t is not None and t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements, got {t.numel()}")


def cov_numel(d_k: int, packed_cov: bool) -> int:
    """Floats per head of the second-moment state: d_k^2, or d_k (d_k + 1) / 2 packed."""
    return d_k * (d_k + 1) // 2 if packed_cov else d_k * d_k


def make_fwd_params(rule, q, k, v, log_alpha, beta, w_lambda, b_lambda, o,
                    carry_in=None, carry_out=None, segments: int = 0, chunk: int = 64,
                    workspace=None, normalize_keys: bool = False, packed_cov: bool = False) -> FwdParams:
    """Fill a ccq_fwd_params from tensors (carry_in / carry_out: (S, C, ksum, n) or None; C is
    [B, H, d_k, d_k], or its packed upper triangle [B, H, d_k (d_k + 1) / 2] with packed_cov)."""
    import torch
    B, H, T, d_k = q.shape
    d_v = v.shape[-1]
    p = FwdParams()
    p.rule = _rule_code(rule)
    p.dtype = _dtype_code(q)
    p.B, p.H, p.T, p.d_k, p.d_v = B, H, T, d_k, d_v
    p.chunk = chunk
    p.segments = segments
    p.flags = _flags(normalize_keys, packed_cov)
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta), ("o", o)):
        _check_dev(name, t, q.dtype)
    _check_dev("w_lambda", w_lambda, torch.float32)
    _check_dev("b_lambda", b_lambda, torch.float32)
    p.q, p.k, p.v, p.log_alpha, p.beta = (_ptr(x) for x in (q, k, v, log_alpha, beta))
    p.w_lambda, p.b_lambda, p.o = _ptr(w_lambda), _ptr(b_lambda), _ptr(o)
    if carry_in is not None:
        S0, C0, m0, n0 = carry_in
        for name, t, dt in (("S0", S0, torch.float32), ("C0", C0, torch.float32),
                            ("ksum0", m0, torch.float32), ("n0", n0, torch.int64)):
            _check_dev(name, t, dt)
        _check_numel("S0", S0, B * H * d_v * d_k)
        _check_numel("C0", C0, B * H * cov_numel(d_k, packed_cov))
        _check_numel("ksum0", m0, B * H * d_k)
        _check_numel("n0", n0, B * H)
        p.S0, p.C0, p.ksum0, p.n0 = _ptr(S0), _ptr(C0), _ptr(m0), _ptr(n0)
    if carry_out is not None:
        S1, C1, m1, n1 = carry_out
        for name, t, dt in (("S_out", S1, torch.float32), ("C_out", C1, torch.float32),
                            ("ksum_out", m1, torch.float32), ("n_out", n1, torch.int64)):
            _check_dev(name, t, dt)
        _check_numel("S_out", S1, B * H * d_v * d_k)
        _check_numel("C_out", C1, B * H * cov_numel(d_k, packed_cov))
        _check_numel("ksum_out", m1, B * H * d_k)
        _check_numel("n_out", n1, B * H)
        p.S_out, p.C_out, p.ksum_out, p.n_out = _ptr(S1), _ptr(C1), _ptr(m1), _ptr(n1)
    if workspace is not None:
        _check_dev("workspace", workspace)
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    return p


def ccq_fwd_workspace_bytes(p: FwdParams) -> int:
    return int(load_library().ccq_fwd_workspace_bytes(ctypes.byref(p)))


def ccq_chunk_carry_bytes(dtype_code: int, B: int, H: int, T: int, d: int) -> int:
    """Bytes of the chunk-carry buffer (ccq_chunk_carry_bytes)."""
    return int(load_library().ccq_chunk_carry_bytes(dtype_code, B, H, T, d))


def new_chunk_carry(q):
    """A chunk-carry buffer (uint8 device tensor) for a prefill / backward of q's shape and dtype."""
    import torch
    B, H, T, d = q.shape
    n = ccq_chunk_carry_bytes(_dtype_code(q), B, H, T, d)
    if n == 0:
        raise ValueError("unsupported shape or dtype for chunk carries")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def ccq_fwd_chunked(rule, q, k, v, log_alpha, beta, w_lambda, b_lambda, o=None,
                    carry_in=None, carry_out=None, segments: int = 0, chunk: int = 64,
                    workspace=None, stream=None, phase_events=None, normalize_keys: bool = False,
                    packed_cov: bool = False, chunk_carry=None):
    """Chunked CCQ prefill through the C ABI.  Allocates o (and the workspace if not
    given) with torch; returns o.  ``phase_events``: optional ctypes array of 4 hipEvent_t
    handles recorded around the kernels of the pass.  ``normalize_keys``: the kernels scale
    every key to unit L2 norm first (CCQ_FLAG_NORMALIZE_KEYS).  ``packed_cov``: the carry's
    C is the packed upper triangle (CCQ_FLAG_PACKED_COV).  ``chunk_carry``: optional buffer
    (``new_chunk_carry``) that receives the carry at every chunk start, for ccq_bwd_chunked."""
    import torch
    lib = load_library()
    if o is None:
        o = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    p = make_fwd_params(rule, q, k, v, log_alpha, beta, w_lambda, b_lambda, o,
                        carry_in, carry_out, segments, chunk, workspace, normalize_keys, packed_cov)
    if workspace is None:
        nbytes = int(lib.ccq_fwd_workspace_bytes(ctypes.byref(p)))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
            p.workspace = workspace.data_ptr()
            p.workspace_bytes = nbytes
    if phase_events is not None:
        p.phase_events = ctypes.cast(phase_events, ctypes.c_void_p)
    if chunk_carry is not None:
        _check_chunk_carry(chunk_carry, q)
        p.chunk_carry = chunk_carry.data_ptr()
    st = lib.ccq_fwd_chunked(ctypes.byref(p), _stream_handle(stream))
    if st != 0:
        raise CcqError(st, "ccq_fwd_chunked")
    return o


def _check_chunk_carry(buf, q):
    _check_dev("chunk_carry", buf)
    B, H, T, d = q.shape
    need = ccq_chunk_carry_bytes(_dtype_code(q), B, H, T, d)
    if buf.numel() * buf.element_size() < need:
        raise ValueError(f"chunk_carry must hold {need} bytes")


def ccq_fwd_chunked_noalloc(rule, q, k, v, log_alpha, beta, w_lambda, b_lambda, o=None,
                            carry_in=None, carry_out=None, segments: int = 0, chunk: int = 64,
                            stream=None, normalize_keys: bool = False, packed_cov: bool = False):
    """ccq_fwd_chunked_noalloc through the C ABI: the prefill with the library's own device array
    as its workspace (nothing is allocated for it; o is allocated here only when not given).
    Returns o."""
    import torch
    lib = load_library()
    if o is None:
        o = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    p = make_fwd_params(rule, q, k, v, log_alpha, beta, w_lambda, b_lambda, o,
                        carry_in, carry_out, segments, chunk, None, normalize_keys, packed_cov)
    st = lib.ccq_fwd_chunked_noalloc(ctypes.byref(p), _stream_handle(stream))
    if st != 0:
        raise CcqError(st, "ccq_fwd_chunked_noalloc")
    return o


def ccq_decode_step(rule, q, k, v, log_alpha, beta, w_lambda, b_lambda, S, C, ksum, n,
                    o=None, stream=None, normalize_keys: bool = False, packed_cov: bool = False):
    """One in-place decode step through the C ABI; returns o [N, H, d_v].  ``normalize_keys``:
    the kernel scales the key to unit L2 norm first (CCQ_FLAG_NORMALIZE_KEYS).  ``packed_cov``:
    C is the packed upper triangle [N, H, d_k (d_k + 1) / 2] (CCQ_FLAG_PACKED_COV)."""
    import torch
    lib = load_library()
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, d_v), dtype=q.dtype, device=q.device)
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta), ("o", o)):
        _check_dev(name, t, q.dtype)
    for name, t, dt in (("w_lambda", w_lambda, torch.float32), ("b_lambda", b_lambda, torch.float32),
                        ("S", S, torch.float32), ("C", C, torch.float32), ("ksum", ksum, torch.float32),
                        ("n", n, torch.int64)):
        _check_dev(name, t, dt)
    _check_numel("S", S, N * H * d_v * d_k)
    _check_numel("C", C, N * H * cov_numel(d_k, packed_cov))
    _check_numel("ksum", ksum, N * H * d_k)
    _check_numel("n", n, N * H)
    st = lib.ccq_decode_step(_rule_code(rule), _dtype_code(q), N, H, d_k, d_v,
                             _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                             _ptr(w_lambda), _ptr(b_lambda), _ptr(S), _ptr(C), _ptr(ksum), _ptr(n),
                             _ptr(o), _flags(normalize_keys, packed_cov), _stream_handle(stream))
    if st != 0:
        raise CcqError(st, "ccq_decode_step")
    return o


def ccq_key_subspace(C, ksum, n, k, r: int = 16, needle=None, packed_cov: bool = False, stream=None,
                     iters=None):
    """Key-covariance subspace diagnostic through the C ABI (see ``ccq_key_subspace`` in ccq.h).
    C [B, H, d, d] (or packed [B, H, d (d + 1) / 2]), ksum [B, H, d], n [B, H] int64: the
    statistics; k [B, H, T, d]: the keys to score; needle [B, H, T] bool / uint8 or None;
    iters: optional int32 [B, H] tensor that receives the bisection work per head (multisection
        rounds summed over the eigenvalues).
    Returns (eigvals [B, H, d], basis [B, H, r, d], align [B, H, T], delta_mu [B, H] or None),
    allocated with torch on k's device."""
    import torch
    lib = load_library()
    B, H, T, d = k.shape
    _check_dev("k", k)
    for name, t, dt in (("C", C, torch.float32), ("ksum", ksum, torch.float32), ("n", n, torch.int64)):
        _check_dev(name, t, dt)
    _check_numel("C", C, B * H * cov_numel(d, packed_cov))
    _check_numel("ksum", ksum, B * H * d)
    _check_numel("n", n, B * H)
    dev = k.device
    eig = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    basis = torch.empty((B, H, r, d), dtype=torch.float32, device=dev)
    align = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    if iters is not None:
        _check_dev("iters", iters, torch.int32)
        _check_numel("iters", iters, B * H)
    dmu = None
    nd = None
    if needle is not None:
        nd = needle.to(torch.uint8).contiguous()
        _check_dev("needle", nd)
        _check_numel("needle", nd, B * H * T)
        dmu = torch.empty((B, H), dtype=torch.float32, device=dev)
    st = lib.ccq_key_subspace(_dtype_code(k), B, H, T, d, r, _ptr(C), _ptr(ksum), _ptr(n), _ptr(k), _ptr(nd),
                              _ptr(eig), _ptr(basis), _ptr(align), _ptr(dmu), _ptr(iters),
                              FLAG_PACKED_COV if packed_cov else 0, _stream_handle(stream))
    if st != 0:
        raise CcqError(st, "ccq_key_subspace")
    return eig, basis, align, dmu


def ccq_step_backward(rule, q, k, v, log_alpha, beta, w_lambda, b_lambda, S, C, ksum, n, d_o, dS, dC, dksum,
                      stream=None):
    """Backward of one recurrence step through the C ABI (see ``ccq_step_backward`` in ccq.h).
    The carry before the step (S, C, ksum, n), the token and d_o are inputs; dS, dC, dksum (fp32)
    hold the adjoint of the carry after the step and are overwritten with the adjoint before it.
    Returns a dict of fp32 tensors: dq, dk, dv, dlog_alpha, dbeta (GDN), dw_lambda [N, H, d_k],
    db_lambda [N, H] (per sequence)."""
    import torch
    lib = load_library()
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta)):
        _check_dev(name, t, q.dtype)
    for name, t, dt in (("w_lambda", w_lambda, torch.float32), ("b_lambda", b_lambda, torch.float32),
                        ("S", S, torch.float32), ("C", C, torch.float32), ("ksum", ksum, torch.float32),
                        ("n", n, torch.int64), ("d_o", d_o, torch.float32), ("dS", dS, torch.float32),
                        ("dC", dC, torch.float32), ("dksum", dksum, torch.float32)):
        _check_dev(name, t, dt)
    for name, t, cnt in (("S", S, N * H * d_v * d_k), ("C", C, N * H * d_k * d_k), ("ksum", ksum, N * H * d_k),
                         ("n", n, N * H), ("d_o", d_o, N * H * d_v), ("dS", dS, N * H * d_v * d_k),
                         ("dC", dC, N * H * d_k * d_k), ("dksum", dksum, N * H * d_k)):
        _check_numel(name, t, cnt)
    rule_c = _rule_code(rule)
    dev = q.device
    f = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((N, H, d_k), **f), dk=torch.empty((N, H, d_k), **f), dv=torch.empty((N, H, d_v), **f),
               dlog_alpha=torch.empty((N, H, d_k) if rule_c == CCQ_RULE_GLA else (N, H), **f),
               dbeta=None if rule_c == CCQ_RULE_GLA else torch.empty((N, H), **f),
               dw_lambda=torch.empty((N, H, d_k), **f), db_lambda=torch.empty((N, H), **f))
    st = lib.ccq_step_backward(rule_c, _dtype_code(q), N, H, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                               _ptr(beta), _ptr(w_lambda), _ptr(b_lambda), _ptr(S), _ptr(C), _ptr(ksum), _ptr(n),
                               _ptr(d_o), _ptr(dS), _ptr(dC), _ptr(dksum), _ptr(out["dq"]), _ptr(out["dk"]),
                               _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]), _ptr(out["dw_lambda"]),
                               _ptr(out["db_lambda"]), 0, _stream_handle(stream))
    if st != 0:
        raise CcqError(st, "ccq_step_backward")
    return out


def ccq_bwd_chunked(rule, q, k, v, log_alpha, w_lambda, b_lambda, d_o, carry_in=None, carry_out_adjoint=None,
                    want_carry_in_adjoint: bool = False, workspace=None, stream=None, phase_events=None, beta=None,
                    chunk_carry=None):
    """Chunked backward of the prefill through the C ABI (see ``ccq_bwd_chunked`` in ccq.h).
    q, k, v, d_o: [B, H, T, d] of one dtype; log_alpha: [B, H, T, d] (GLA) or [B, H, T] (Gated
    DeltaNet, with beta [B, H, T]); carry_in: (S0, C0, ksum0, n0) or None; carry_out_adjoint:
    (dS_T, dC_T, dksum_T) fp32 or None.  Returns a dict of fp32 tensors dq, dk, dv, dlog_alpha (the
    shape of log_alpha), dbeta (Gated DeltaNet), dw_lambda [B, H, d], db_lambda [B, H] and, with
    want_carry_in_adjoint, dS0, dC0, dksum0.  ``phase_events``: optional ctypes array of 5
    hipEvent_t handles recorded around the passes.  ``chunk_carry``: the buffer a ccq_fwd_chunked of
    the same inputs filled; the chunk carries are then read from it instead of recomputed."""
    import torch
    lib = load_library()
    B, H, T, d_k = q.shape
    d_v = v.shape[-1]
    rule_c = _rule_code(rule)
    gdn = rule_c == CCQ_RULE_GDN
    if gdn != (beta is not None):
        raise ValueError("beta is given for Gated DeltaNet and only for it")
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("d_o", d_o), ("beta", beta)):
        _check_dev(name, t, q.dtype)
        per = d_v if name in ("v", "d_o") else (1 if name == "beta" or (gdn and name == "log_alpha") else d_k)
        _check_numel(name, t, B * H * T * per)
    _check_dev("w_lambda", w_lambda, torch.float32)
    _check_dev("b_lambda", b_lambda, torch.float32)
    p = BwdParams()
    p.rule = rule_c
    p.dtype = _dtype_code(q)
    p.B, p.H, p.T, p.d_k, p.d_v, p.chunk = B, H, T, d_k, d_v, 64
    p.q, p.k, p.v, p.log_alpha, p.d_o = (_ptr(x) for x in (q, k, v, log_alpha, d_o))
    p.w_lambda, p.b_lambda = _ptr(w_lambda), _ptr(b_lambda)
    if carry_in is not None:
        S0, C0, m0, n0 = carry_in
        for name, t, dt, cnt in (("S0", S0, torch.float32, B * H * d_v * d_k), ("C0", C0, torch.float32, B * H * d_k * d_k),
                                 ("ksum0", m0, torch.float32, B * H * d_k), ("n0", n0, torch.int64, B * H)):
            _check_dev(name, t, dt)
            _check_numel(name, t, cnt)
        p.S0, p.C0, p.ksum0, p.n0 = _ptr(S0), _ptr(C0), _ptr(m0), _ptr(n0)
    if carry_out_adjoint is not None:
        dS_T, dC_T, dm_T = carry_out_adjoint
        for name, t, cnt in (("dS_T", dS_T, B * H * d_v * d_k), ("dC_T", dC_T, B * H * d_k * d_k),
                             ("dksum_T", dm_T, B * H * d_k)):
            _check_dev(name, t, torch.float32)
            _check_numel(name, t, cnt)
        p.dS_T, p.dC_T, p.dksum_T = _ptr(dS_T), _ptr(dC_T), _ptr(dm_T)
    f = dict(dtype=torch.float32, device=q.device)
    out = dict(dq=torch.empty((B, H, T, d_k), **f), dk=torch.empty((B, H, T, d_k), **f),
               dv=torch.empty((B, H, T, d_v), **f),
               dlog_alpha=torch.empty((B, H, T) if gdn else (B, H, T, d_k), **f),
               dw_lambda=torch.empty((B, H, d_k), **f), db_lambda=torch.empty((B, H), **f))
    if gdn:
        out["dbeta"] = torch.empty((B, H, T), **f)
        p.beta, p.dbeta = _ptr(beta), _ptr(out["dbeta"])
    if want_carry_in_adjoint:
        out.update(dS0=torch.empty((B, H, d_v, d_k), **f), dC0=torch.empty((B, H, d_k, d_k), **f),
                   dksum0=torch.empty((B, H, d_k), **f))
        p.dS0, p.dC0, p.dksum0 = _ptr(out["dS0"]), _ptr(out["dC0"]), _ptr(out["dksum0"])
    p.dq, p.dk, p.dv, p.dlog_alpha = _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"])
    p.dw_lambda, p.db_lambda = _ptr(out["dw_lambda"]), _ptr(out["db_lambda"])
    nbytes = int(lib.ccq_bwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_dev("workspace", workspace)
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    if phase_events is not None:
        p.phase_events = ctypes.cast(phase_events, ctypes.c_void_p)
    if chunk_carry is not None:
        _check_chunk_carry(chunk_carry, q)
        p.chunk_carry = chunk_carry.data_ptr()
    st = lib.ccq_bwd_chunked(ctypes.byref(p), _stream_handle(stream))
    if st != 0:
        raise CcqError(st, "ccq_bwd_chunked")
    return out

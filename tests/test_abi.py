"""The C ABI library loads, exports what include/ccq.h declares, and rejects bad
arguments with the documented status codes before enqueuing anything.  No call
here reaches a kernel, so these run without a GPU."""

import ctypes
import os
import re

import pytest

from curvature_conditioned_query_amd import binding
from curvature_conditioned_query_amd.binding import BwdParams, FwdParams, load_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ccq.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, LAUNCH, WORKSPACE = 0, -1, -2, -3, -4, -5
FAKE = 0x7F0000000000  # aligned, never dereferenced: every case below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ccq_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTED_SYMBOLS)
    for name in names:
        assert hasattr(lib, name), f"libccq.so does not export {name}"
    assert lib.ccq_abi_version() == 11


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, MISALIGNED, LAUNCH, WORKSPACE, 17):
        s = lib.ccq_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0


def _params(**kw):
    p = FwdParams()
    p.rule, p.dtype, p.B, p.H, p.T, p.d_k, p.d_v, p.chunk = 0, 1, 1, 2, 256, 128, 128, 64
    p.q = p.k = p.v = p.log_alpha = p.w_lambda = p.b_lambda = p.o = FAKE
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _fwd(lib, p):
    return lib.ccq_fwd_chunked(ctypes.byref(p), None)


@pytest.mark.parametrize("kw,code", [
    (dict(rule=7), INVALID), (dict(dtype=5), INVALID), (dict(B=0), INVALID), (dict(H=-1), INVALID),
    (dict(T=0), INVALID), (dict(chunk=32), UNSUPPORTED), (dict(d_k=96, d_v=96), UNSUPPORTED),
    (dict(d_k=64, d_v=128), UNSUPPORTED), (dict(dtype=0), UNSUPPORTED), (dict(q=None), INVALID),
    (dict(o=None), INVALID), (dict(beta=FAKE), INVALID), (dict(rule=1), INVALID),
    (dict(S0=FAKE), INVALID), (dict(S_out=FAKE, C_out=FAKE), INVALID), (dict(k=FAKE + 4), MISALIGNED),
    (dict(segments=-2), INVALID), (dict(flags=4), INVALID), (dict(flags=-1), INVALID),
])
def test_fwd_argument_errors(lib, kw, code):
    assert _fwd(lib, _params(**kw)) == code
    assert lib.ccq_fwd_workspace_bytes(ctypes.byref(_params(**kw))) == 0


def test_fwd_null_params(lib):
    assert lib.ccq_fwd_chunked(None, None) == INVALID
    assert lib.ccq_fwd_workspace_bytes(None) == 0


def test_fwd_workspace_sizing_and_check(lib):
    p = _params(B=4, H=16, T=4096)
    need = lib.ccq_fwd_workspace_bytes(ctypes.byref(p))
    assert need > 0  # 64 chains < 256 target groups: segments in use
    # too small a workspace is refused before launch
    p.workspace, p.workspace_bytes = FAKE, need - 16
    assert _fwd(lib, p) == WORKSPACE
    p.workspace = None
    assert _fwd(lib, p) == WORKSPACE
    # one segment per chain needs none
    assert lib.ccq_fwd_workspace_bytes(ctypes.byref(_params(B=4, H=16, T=4096, segments=1))) == 0
    assert lib.ccq_fwd_workspace_bytes(ctypes.byref(_params(B=64, H=16, T=64))) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(rule=7), INVALID), (dict(B=0), INVALID), (dict(chunk=32), UNSUPPORTED), (dict(q=None), INVALID),
    (dict(k=FAKE + 4), MISALIGNED), (dict(flags=4), INVALID), (dict(S0=FAKE), INVALID),
])
def test_fwd_noalloc_argument_errors(lib, kw, code):
    """The no-allocation variant validates exactly as ccq_fwd_chunked does, before any HIP call."""
    assert lib.ccq_fwd_chunked_noalloc(ctypes.byref(_params(**kw)), None) == code
    assert lib.ccq_fwd_chunked_noalloc(None, None) == INVALID


def test_fwd_noalloc_rejects_segments_beyond_its_array(lib):
    """An explicit segment count whose workspace exceeds the 64 MiB array is refused before any
    launch; the workspace fields are ignored (no workspace is needed or read)."""
    scratch = 64 << 20
    # Gated DeltaNet slots are 3 d^2 + d floats: 256 chains x 4 segments x 197,120 B > 64 MiB
    p = _params(rule=1, beta=FAKE, B=16, H=16, T=4096, segments=4)
    assert lib.ccq_fwd_workspace_bytes(ctypes.byref(p)) > scratch
    assert lib.ccq_fwd_chunked_noalloc(ctypes.byref(p), None) == WORKSPACE
    p.workspace, p.workspace_bytes = FAKE, 1 << 40  # a caller workspace does not help: it is not used
    assert lib.ccq_fwd_chunked_noalloc(ctypes.byref(p), None) == WORKSPACE


def _dec(lib, rule=0, dtype=1, N=2, H=2, dk=128, dv=128, flags=0, **ptrs):
    names = ["q", "k", "v", "log_alpha", "beta", "w_lambda", "b_lambda", "S", "C", "ksum", "n", "o"]
    vals = {n: FAKE for n in names}
    vals["beta"] = None if rule == 0 else FAKE
    vals.update(ptrs)
    return lib.ccq_decode_step(rule, dtype, N, H, dk, dv, *[vals[n] for n in names], flags, None)


@pytest.mark.parametrize("kw,code", [
    (dict(rule=3), INVALID), (dict(dtype=2), INVALID), (dict(N=0), INVALID), (dict(H=0), INVALID),
    (dict(dk=32, dv=32), UNSUPPORTED), (dict(dk=128, dv=64), UNSUPPORTED), (dict(q=None), INVALID),
    (dict(S=None), INVALID), (dict(n=None), INVALID), (dict(beta=FAKE), INVALID),
    (dict(rule=1, beta=None), INVALID), (dict(C=FAKE + 8), MISALIGNED), (dict(flags=4), INVALID), (dict(flags=8), INVALID),
])
def test_decode_argument_errors(lib, kw, code):
    assert _dec(lib, **kw) == code


def _sub(lib, dtype=1, B=2, H=2, T=100, dk=128, r=16, flags=0, **ptrs):
    names = ["C", "ksum", "n", "k", "needle", "eigvals", "basis", "align", "delta_mu", "iters"]
    vals = {n: FAKE for n in names}
    vals["iters"] = None
    vals.update(ptrs)
    return lib.ccq_key_subspace(dtype, B, H, T, dk, r, *[vals[n] for n in names], flags, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), INVALID), (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(r=0), INVALID),
    (dict(dk=64, r=65), INVALID), (dict(r=33), UNSUPPORTED), (dict(dk=96, r=8), UNSUPPORTED),
    (dict(B=300, H=300), UNSUPPORTED), (dict(C=None), INVALID), (dict(k=None), INVALID),
    (dict(basis=None), INVALID), (dict(align=None), INVALID), (dict(needle=None), INVALID),
    (dict(delta_mu=None), INVALID), (dict(flags=1), INVALID), (dict(flags=4), INVALID),
    (dict(ksum=FAKE + 4), MISALIGNED), (dict(needle=FAKE + 1), MISALIGNED), (dict(iters=FAKE + 4), MISALIGNED),
])
def test_subspace_argument_errors(lib, kw, code):
    assert _sub(lib, **kw) == code


def _sb(lib, rule=0, dtype=1, N=2, H=2, dk=128, dv=128, flags=0, **ptrs):
    names = ["q", "k", "v", "log_alpha", "beta", "w_lambda", "b_lambda", "S", "C", "ksum", "n", "d_o", "dS", "dC",
             "dksum", "dq", "dk", "dv", "dlog_alpha", "dbeta", "dw_lambda", "db_lambda"]
    vals = {n: FAKE for n in names}
    if rule == 0:
        vals["beta"] = vals["dbeta"] = None
    vals.update(ptrs)
    return lib.ccq_step_backward(rule, dtype, N, H, dk, dv, *[vals[n] for n in names], flags, None)


@pytest.mark.parametrize("kw,code", [
    (dict(rule=2), INVALID), (dict(dtype=9), INVALID), (dict(N=0), INVALID), (dict(dk=64, dv=64), UNSUPPORTED),
    (dict(dk=128, dv=64), UNSUPPORTED), (dict(flags=1), UNSUPPORTED), (dict(flags=2), UNSUPPORTED),
    (dict(flags=4), INVALID), (dict(q=None), INVALID), (dict(d_o=None), INVALID), (dict(dS=None), INVALID),
    (dict(dw_lambda=None), INVALID), (dict(beta=FAKE), INVALID), (dict(dbeta=FAKE), INVALID),
    (dict(rule=1, beta=None, dbeta=FAKE), INVALID), (dict(rule=1, beta=FAKE, dbeta=None), INVALID),
    (dict(dC=FAKE + 4), MISALIGNED),
])
def test_step_backward_argument_errors(lib, kw, code):
    # every case must fail validation: a call that passed it would launch on the fake pointers
    assert code != OK
    assert _sb(lib, **kw) == code


def _bparams(**kw):
    p = BwdParams()
    p.rule, p.dtype, p.B, p.H, p.T, p.d_k, p.d_v, p.chunk = 0, 1, 2, 2, 200, 128, 128, 64
    for n in ("q", "k", "v", "log_alpha", "w_lambda", "b_lambda", "d_o", "dq", "dk", "dv", "dlog_alpha",
              "dw_lambda", "db_lambda"):
        setattr(p, n, FAKE)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,code", [
    (dict(rule=5), INVALID), (dict(rule=1), INVALID), (dict(rule=1, beta=FAKE), INVALID),
    (dict(rule=1, dbeta=FAKE), INVALID), (dict(beta=FAKE, dbeta=FAKE), INVALID),
    (dict(rule=1, beta=FAKE + 2, dbeta=FAKE), MISALIGNED), (dict(dtype=3), INVALID), (dict(T=0), INVALID),
    (dict(B=-1), INVALID), (dict(chunk=-1), INVALID), (dict(chunk=128), UNSUPPORTED), (dict(flags=1), UNSUPPORTED),
    (dict(flags=2), UNSUPPORTED), (dict(flags=8), INVALID), (dict(d_k=64, d_v=128), UNSUPPORTED),
    (dict(dtype=0), UNSUPPORTED), (dict(d_k=256, d_v=256), UNSUPPORTED), (dict(B=300, H=300), UNSUPPORTED),
    (dict(q=None), INVALID), (dict(d_o=None), INVALID), (dict(dlog_alpha=None), INVALID),
    (dict(db_lambda=None), INVALID), (dict(S0=FAKE), INVALID), (dict(dS_T=FAKE, dC_T=FAKE), INVALID),
    (dict(dS0=FAKE), INVALID), (dict(dv=FAKE + 8), MISALIGNED), (dict(n0=FAKE + 4, S0=FAKE, C0=FAKE, ksum0=FAKE), MISALIGNED),
])
def test_bwd_argument_errors(lib, kw, code):
    # every case must fail validation: a call that passed it would launch on the fake pointers
    assert code != OK
    p = _bparams(**kw)
    assert lib.ccq_bwd_chunked(ctypes.byref(p), None) == code
    assert lib.ccq_bwd_workspace_bytes(ctypes.byref(p)) == 0


def test_bwd_workspace_sizing_and_check(lib):
    assert lib.ccq_bwd_chunked(None, None) == INVALID
    assert lib.ccq_bwd_workspace_bytes(None) == 0
    p = _bparams(B=4, H=16, T=4096)
    need = lib.ccq_bwd_workspace_bytes(ctypes.byref(p))
    # per chain and chunk (bf16): the fp32 carry update (2 d^2 + 2 d), the bf16 carry and adjoint
    # matrices (2 d^2 each), the fp32 key sum (d) and adjoint tails (4 d), three fp32 [64, d] tiles
    d = 128
    per = (2 * d * d + 2 * d) * 4 + 2 * d * d * 2 + d * 4 + 2 * d * d * 2 + 4 * d * 4 + 3 * 64 * d * 4
    assert need == 4 * 16 * 64 * per
    p.workspace, p.workspace_bytes = FAKE, need - 16
    assert lib.ccq_bwd_chunked(ctypes.byref(p), None) == WORKSPACE
    p.workspace = None
    assert lib.ccq_bwd_chunked(ctypes.byref(p), None) == WORKSPACE


def test_gdn_bwd_workspace_sizing(lib):
    """Gated DeltaNet: the prefill's segment slots for the carry pass (about one segment per compute
    unit: 4 per chain at 64 chains), then per chain and chunk (bf16) the bf16 carry and adjoint
    matrices (2 d^2 each), the fp32 key sum (d) and adjoint tails (4 d), the bf16 64 x 64 triangular
    inverse and two fp32 [64, d] tiles."""
    p = _bparams(rule=1, beta=FAKE, dbeta=FAKE, B=4, H=16, T=4096)
    need = lib.ccq_bwd_workspace_bytes(ctypes.byref(p))
    d, chains, P = 128, 64, 4
    seg = chains * P * (3 * d * d + d) * 4 + chains * 8
    seg = (seg + 255) // 256 * 256
    per = 2 * d * d * 2 + d * 4 + 64 * 64 * 2 + 2 * d * d * 2 + 4 * d * 4 + 2 * 64 * d * 4
    assert need == seg + chains * 64 * per
    p.workspace, p.workspace_bytes = FAKE, need - 16
    assert lib.ccq_bwd_chunked(ctypes.byref(p), None) == WORKSPACE



def test_chunk_carry_bytes(lib):
    """B H ceil(T / 64) (2 d^2 sizeof(dtype) + 4 d); 0 for what the chunked calls reject."""
    f = lib.ccq_chunk_carry_bytes
    assert f(1, 4, 16, 4096, 128) == 64 * 64 * (2 * 128 * 128 * 2 + 4 * 128)
    assert f(0, 1, 2, 200, 64) == 2 * 4 * (2 * 64 * 64 * 4 + 4 * 64)
    assert f(1, 1, 1, 65, 64) == 2 * (2 * 64 * 64 * 2 + 4 * 64)
    for args in ((2, 1, 1, 64, 64), (1, 0, 1, 64, 64), (1, 1, 1, 0, 64), (1, 1, 1, 64, 96), (0, 1, 1, 64, 128)):
        assert f(*args) == 0


def test_chunk_carry_must_be_aligned(lib):
    p = _params(chunk_carry=FAKE + 8)
    assert _fwd(lib, p) == MISALIGNED
    b = BwdParams()
    b.rule, b.dtype, b.B, b.H, b.T, b.d_k, b.d_v, b.chunk = 0, 1, 1, 2, 256, 128, 128, 64
    for name in ("q", "k", "v", "log_alpha", "w_lambda", "b_lambda", "d_o", "dq", "dk", "dv", "dlog_alpha",
                 "dw_lambda", "db_lambda"):
        setattr(b, name, FAKE)
    b.chunk_carry = FAKE + 8
    assert lib.ccq_bwd_chunked(ctypes.byref(b), None) == MISALIGNED


def test_param_structs_match_the_header(tmp_path):
    """Every field of the ctypes mirrors sits where the C compiler puts it, and the sizes agree."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "ccq.h"', "int main(void) {"]
    for cname, cls in (("ccq_fwd_params", FwdParams), ("ccq_bwd_params", BwdParams)):
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            cname, field, value = line.split()
            got[(cname, field)] = int(value)
    for cname, cls in (("ccq_fwd_params", FwdParams), ("ccq_bwd_params", BwdParams)):
        assert got[(cname, "size")] == ctypes.sizeof(cls)
        for field, _ in cls._fields_:
            assert got[(cname, field)] == getattr(cls, field).offset, (cname, field)

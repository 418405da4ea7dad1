"""Build libccq.so in-tree with hipcc for gfx950.

    python -m curvature_conditioned_query_amd.build [--jobs N]

Every source is compiled on each call (no reuse of stale objects), one hipcc per
translation unit in parallel, then linked into ``curvature_conditioned_query_amd/libccq.so``.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libccq.so")
SOURCES = ["ccq_api.cpp", "ccq_decode.hip", "ccq_decode_packed.hip", "ccq_prefill.hip", "ccq_prefill_summary.hip", "ccq_prefill_gdn.hip", "ccq_prefill_gdn_summary.hip", "ccq_prefill_pipe.hip", "ccq_subspace.hip",
           "ccq_step_backward.hip", "ccq_backward.hip", "ccq_backward_gdn.hip", "ccq_noalloc.hip"]
ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]
# Per-source scheduler choice, measured on the GPU against the default: the GLA prefill's main
# kernel is 2-3 % faster with the iterative ILP scheduler; its segment summary and carry scan are
# 3 % faster under the max-ILP one (and 1-3 % slower under iterative ILP), so they sit in a file
# of their own.  The Gated DeltaNet kernels spill far more under iterative ILP and keep the
# default.
# The full-C decode step moves its 1 GiB of state 5 % faster under the same scheduler (6.23 against
# 5.91 TB/s); the packed-C variants are 8 % slower under it, so they sit in a file of their own.
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
# The Gated DeltaNet segment summary is faster under the memory-clause scheduler, its main kernel
# slower, so the summary is instantiated in a file of its own.
EXTRA = {"ccq_prefill.hip": _ILP, "ccq_decode.hip": _ILP,
         "ccq_prefill_summary.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
         "ccq_prefill_gdn_summary.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}


def library_sha256() -> str:
    """sha256 over everything that decides the built code: every file under csrc/ and include/
    (name and contents, in sorted order) and the compile flags of every translation unit.
    Counter records under profiles/ store it, so a record stops counting as soon as any
    source, header or flag changes."""
    import hashlib
    h = hashlib.sha256()
    for top in (CSRC, INCLUDE):
        for name in sorted(os.listdir(top)):
            path = os.path.join(top, name)
            if os.path.isfile(path):
                h.update(os.path.relpath(path, ROOT).encode())
                with open(path, "rb") as f:
                    h.update(f.read())
    # the flags name the include directories by absolute path: hash them relative to the repository
    # root, so that the same tree gives the same hash wherever it is checked out
    for src in SOURCES:
        flags = [f.replace(ROOT, "<root>") for f in (src, *COMMON, *DEVICE_FLAGS, *EXTRA.get(src, []))]
        h.update(" ".join(flags).encode())
    return h.hexdigest()


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 0, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

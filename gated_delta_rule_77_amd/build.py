"""Compile libpdn.so for gfx950 in-tree with hipcc.

Each source compiles to its own object under ``_build/`` (in parallel), then
one shared library is linked next to this file.  Every HIP source is built
with packed-fp32 instructions disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpdn.so")
ARCH = os.environ.get("PDN_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
          "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


# Per-source extra flags.  The prefill kernels keep their MFMA accumulators in
# ordinary VGPRs (no accumulator-register copies around every VALU use).  The
# kernels that the *_ilp.hip sources instantiate are scheduled for
# instruction-level parallelism: the same operations and results, reordered.
# That made the backward's gradient kernel and 32-column state passes 2-4%
# faster and the per-channel-gate preparation kernel with symmetric keys and
# per-channel decay and gain 3% faster; the other kernels measured equal or
# slower with it (that preparation kernel 10-20% slower with asymmetric keys or
# the stabilised preconditioner).
ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {"chunk_fact.hip": VGPR_FORM,
         "chunk_vec.hip": VGPR_FORM,
         "chunk_vec_ilp.hip": VGPR_FORM + ILP,
         "chunk_bwd_ilp.hip": ILP}


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpdn.so")
    return p


def sources():
    out = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip") or f.endswith(".cpp"):
            out.append(os.path.join(CSRC, f))
    return out


def _compile(src: str, hipcc: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc, *COMMON, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    if verbose:
        noise = "not a recognized feature"
        msg = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if msg.strip():
            print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link libpdn.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each source is compiled to an object under _build/ in parallel, then linked
into expert_routed_ffn_amd/libmoe.so.  Runs on a machine without a GPU.
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
LIB = os.path.join(PKG, "libmoe.so")

SOURCES = ["api.hip", "route_topk.hip", "dispatch.hip", "ffn_gemv.hip", "ffn_mfma.hip", "combine.hip",
           "slot_table.hip", "router.hip", "noalloc.hip"]

ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for all device code.  Floating-point
# contraction is off: a multiply and an add are fused only where the source asks
# for it (__builtin_fmaf).  With contraction left to the compiler, two compiled
# instances of the same code (e.g. kernels specialised for different token
# counts) were measured to round differently, which breaks bit-identical results
# between entry points that share arithmetic.
CFLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-ffp-contract=off", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


# The host pass of hipcc does not know the device-only feature named in CFLAGS
# and says so once per file; that line carries no information.
_HOST_FEATURE_NOTE = "packed-fp32-ops' is not a recognized feature"


def _diagnostics(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if _HOST_FEATURE_NOTE not in l and l.strip())


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    diag = _diagnostics(r.stdout + "\n" + r.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{diag}")
    if diag:  # real warnings stay visible
        print(f"hipcc {src}:\n{diag}", file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

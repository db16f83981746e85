"""Build the HIP library ``libattn_mi355x.so`` in-tree for gfx950.

Usage: ``python -m attention_forward_backward_amd.build`` (or call ``build()``).
Compiles every ``csrc/*.hip`` to an object in ``_build/`` (in parallel), then
links them into ``attention_forward_backward_amd/libattn_mi355x.so``.  Always
recompiles: the result must match the sources.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn_mi355x.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed f32 VALU ops.
# -amdgpu-mfma-vgpr-form: MFMA results in ordinary VGPRs, so the softmax VALU
# reads them without accumulator-register copies.
# -fno-honor-nans: no value on these paths is a NaN (inputs are finite and
# masked scores are -inf), so maxima need no NaN-quieting of MFMA results.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans",
    "-I", os.path.join(ROOT, "include"),
]
# Per-source additions.  The f32 dK+dV kernel (D <= 64) is asked to fit two
# waves per SIMD (256 registers); LLVM's ILP-first scheduler is the one that
# meets that bound without spilling, so its source uses it.  The few-query
# forward needs every load of an iteration issued before the first use; the
# default scheduler interleaves them with the arithmetic and waits for each.
FILE_FLAGS = {
    "attn_bwd_dkdv.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "attn_fwd_small.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the attention library needs the ROCm toolchain")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src,
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = list(extra_flags or [])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])

"""Build ``libhad.so`` (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m binarized_qk_sparse_amd.build

Each source is compiled to an object in ``_build/`` (in parallel), then linked
into ``binarized_qk_sparse_amd/libhad.so``.  ``libhad_ubench.so`` (the measured
VALU and v_exp ceilings that bench.py reports beside the datasheet peaks) is
linked from ``ubench.hip`` alone.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhad.so")
SOURCES = ["api.cpp", "pack.hip", "vquant.hip", "topn.hip", "topn_mfma.hip", "topn_stream.hip", "dense_q8.hip",
           "noalloc.hip", "dense_long.hip", "topn_wide.hip"]
UBENCH_LIB = os.path.join(PKG, "libhad_ubench.so")
UBENCH_SOURCES = ["ubench.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-fPIC",
        "-std=c++17",
        "-ffp-contract=off",
        "-munsafe-fp-atomics",
        # packed fp32 VALU ops stay off: plain v_fma_f32 / v_add_f32 only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core results and accumulators in VGPRs: no accumulator-register copies
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wall",
        "-Wno-unused-function",
        f"-I{os.path.join(ROOT, 'include')}",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(lib: str, objs) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + UBENCH_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(LIB, objs[: len(SOURCES)])
    _link(UBENCH_LIB, objs[len(SOURCES):])
    if verbose:
        print(f"built {LIB} and {os.path.basename(UBENCH_LIB)}")
    return LIB


if __name__ == "__main__":
    build()

"""Compile libmesa.so (HIP, gfx950) in-tree with hipcc.

Every call recompiles.  Objects go to test_regression_amd/_build/, the shared
library to test_regression_amd/libmesa.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmesa.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
SOURCES = ["mesa_host.hip", "chunk_states.hip", "cg_output.hip", "cg_output_bf16.hip", "decode.hip", "qk_preprocess.hip",
           "bwd_adjoint.hip", "bwd_states.hip", "bwd_kv.hip", "bwd_gate.hip", "hawk.hip", "probes.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


# Per-source additions.  The probes' plain accumulator loops are allocated
# with tied accumulator chains only in the VGPR form of MFMA (the AGPR form
# shuffles them through copies); the other kernels are cleanest in the
# default form.  (The bf16-input CG kernels ran 3-4% faster in the VGPR
# form, but there the compiler gives some MFMAs an accumulator input that is
# rewritten a few wait states later, the pattern codegen_check rejects.)
SOURCE_FLAGS = {"probes.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def flags_for(src: str):
    return [*FLAGS, *SOURCE_FLAGS.get(src, [])]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

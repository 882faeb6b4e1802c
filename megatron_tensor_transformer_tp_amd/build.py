"""Build the gfx950 shard library in-tree: ``libtp_shard.so`` next to this file.

Each source is compiled by its own ``hipcc`` process (in parallel), then the
objects are linked into one shared library.  Usage::

    python -m megatron_tensor_transformer_tp_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libtp_shard.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = [
    "tp_shard_abi.cpp",
    "gemm_bf16.hip",
    "gemm_bf16_256_gelu.hip",
    "gemm_bf16_256_plain.hip",
    "gemm_bf16_128_gelu.hip",
    "gemm_bf16_128_plain.hip",
    "gemm_bf16_64_gelu.hip",
    "gemm_bf16_64_plain.hip",
    "gemm_bf16_384_gelu.hip",
    "gemm_bf16_384_plain.hip",
    "gemm_bf16_256_nt.hip",
    "gemm_bf16_256_tn.hip",
    "gemm_bf16_128_nt.hip",
    "gemm_bf16_128_tn.hip",
    "gemm_bf16_256_swiglu.hip",
    "gemm_bf16_128_swiglu.hip",
    "gemm_f32.hip",
    "colsum.hip",
    "sp_reduce.hip",
    "gelu.hip",
    "attention.hip",
    "noalloc.hip",
    "splitk.hip",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    if os.path.exists(obj):
        os.remove(obj)  # a failed compile must never leave a stale object to link
    cmd = [HIPCC, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source for gfx950 and link ``libtp_shard.so``; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    if os.path.exists(LIB_PATH):
        os.remove(LIB_PATH)  # a failed build leaves no library: loading then fails loudly
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build the gfx950 HIP library libfp8mlp.so in-tree with hipcc.

Usage: python -m fp8_tensorwise_scaled_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8mlp.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["quant.hip", "gemm.hip", "gemm_nt_fast.hip", "gemm_nt_exact.hip", "gemm_nn_fast.hip",
           "gemm_nn_exact.hip", "gemm_tn_fast.hip", "gemm_tn_exact.hip", "lm_head_ce.hip",
           "muon.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          # packed fp32 VALU ops stay off (v_pk_*_f32)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, "-I", os.path.join(HERE, "..", "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4, 16)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # Resolve every symbol now, in a child process: a kernel template whose
    # host pass failed silently leaves its launch stub undefined, which would
    # otherwise surface only when the library is first loaded.
    chk = subprocess.run([sys.executable, "-c", "import ctypes, os, sys; ctypes.CDLL(sys.argv[1], mode=os.RTLD_NOW)",
                          tmp], capture_output=True, text=True)
    if chk.returncode != 0:
        os.remove(tmp)
        raise RuntimeError(f"built library does not load:\n{chk.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

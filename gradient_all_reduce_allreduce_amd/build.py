"""Compile the HIP library ``libddp_allreduce.so`` in-tree for gfx950.

    python -m gradient_all_reduce_allreduce_amd.build              # the library
    python -m gradient_all_reduce_allreduce_amd.build --patterns   # hbm_patterns only

The HBM access-pattern benchmark (``csrc/hbm_patterns.hip``, a standalone
measurement program, not part of the library) has its own command, so that
the library build never depends on it.

Every source is compiled by hipcc for gfx950 only, with
  -ffp-contract=off      no fused multiply-add anywhere (results are defined
                         with one rounding per operation)
  packed-fp32-ops off    no packed float32 instructions
and without fast-math or flushing of subnormals.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libddp_allreduce.so")
PATTERNS = os.path.join(PKG, "hbm_patterns")     # HBM access-pattern benchmark
SOURCES = ["api.cpp", "ring_reduce.hip", "ring_reduce_f32_f32.hip",
           "ring_reduce_f32_bf16.hip", "ring_reduce_bf16_f32.hip",
           "ring_reduce_bf16_bf16.hip", "ring_allgather.hip", "ring_step.hip",
           "multi_tensor.hip", "bucket_copy.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]
DEVICE = [f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_patterns(verbose=False):
    """Compile the HBM access-pattern benchmark to ``hbm_patterns``."""
    cmd = [HIPCC, *COMMON, *DEVICE, os.path.join(CSRC, "hbm_patterns.hip"), "-o",
           PATTERNS + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(PATTERNS + ".tmp", PATTERNS)
    if verbose:
        print(f"built {PATTERNS}")
    return PATTERNS


def build(verbose=False):
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    if "--patterns" in sys.argv[1:]:
        build_patterns(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)

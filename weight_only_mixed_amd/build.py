"""Build libslq.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libslq.so")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          # never let the compiler form packed fp32 ops
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-source extra flags: quantization must be bit-exact IEEE (no contraction)
EXTRA = {"quantize.hip": ["-ffp-contract=off"],
         # GPTQ's column pass matches the oracle operation for operation: every
         # fused multiply-add is written out, nothing else may be contracted
         "gptq.hip": ["-ffp-contract=off"],
         # MFMA results in VGPRs: the decode epilogue reads them with plain VALU ops
         "gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
SOURCES = ["quantize.hip", "gemv.hip", "gemm.hip", "fidelity.hip", "mckp.hip", "gptq.hip", "probe.hip",
           "noalloc.hip",
           "slq_abi.cpp"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = ["hipcc", "-x", "hip", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

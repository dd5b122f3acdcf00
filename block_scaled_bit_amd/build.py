"""Build libbsb.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m block_scaled_bit_amd.build

Flags that matter for the numerics:
  * no fast-math: the quantisation divides must be IEEE correctly rounded
    (hipcc's default for float division), and rint must stay half-to-even;
  * -ffp-contract=off: the only fused multiply-adds are the explicit ones in
    the per-group epilogue;
  * -fno-gpu-flush-denormals-to-zero: subnormal scales are honoured;
  * packed-FP32 VALU instructions are disabled (plain v_fma_f32 / v_mul_f32).
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
LIB = os.path.join(PKG, "libbsb.so")
SOURCES = ["quant.hip", "decode.hip", "gemm.hip", "gemm_big.hip", "gemm_mid.hip", "gemm_a16.hip", "gemm_packed.hip", "moe.hip", "attn.hip", "probe.hip", "api.cpp"]
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libbsb")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]   # src may be absolute
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the GPU target feature; that warning is harmless
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(extra=(), verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)

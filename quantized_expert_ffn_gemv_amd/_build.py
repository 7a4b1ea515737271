"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled to an object in parallel, then linked
into quantized_expert_ffn_gemv_amd/libmoe.so.  Usage: ``python -m
quantized_expert_ffn_gemv_amd._build`` or ``build()`` from Python.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    f"-I{INCLUDE}", f"-I{CSRC}",
    # keep float32 arithmetic on plain (non-packed) VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source flags.  The decode kernels keep their few MFMA accumulators in
# VGPRs, which saves an accumulator-register read per result element.
PER_FILE = {
    "ffn_dec.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # The grouped GEMM runs one workgroup per CU (two waves per SIMD, its LDS
    # ring takes most of the CU's LDS): schedule for latency, so each LDS
    # operand read is issued ahead of the MFMAs that precede its use.
    "ffn_gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libmoe.so.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)

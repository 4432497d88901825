"""Compile the HIP sources in csrc/ into libgptq_mi355x.so (gfx950 only).

    python -m post_weight_quantization_14_amd.build [-v]

Objects go to <repo>/_build/, the shared library next to this file so that it
ships with the package tree.  Always recompiles (it is the build check).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgptq_mi355x.so")
SOURCES = ("abi.hip", "gemm_f32.hip", "hessian.hip", "prepare.hip", "quantize.hip", "rtn.hip", "w4a16.hip", "awq.hip", "gemm_x6.hip", "checkpoint.hip",
           *(f"block_quant_g{g}.hip" for g in (0, 8, 16, 32, 64, 128)))

HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ops stay off: the compiler may not form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", SRC,
]
# per-source additions: the W4A16 product keeps its MFMA accumulators in
# ordinary VGPRs (they are read by VALU code after every group; in AGPRs each
# read is a v_accvgpr_read first)
EXTRA = {"w4a16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(SRC, src), "-o", obj]
    t0 = time.time()
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{err}")
    if verbose:
        print(f"  {src}: {time.time() - t0:.1f}s" + (f"\n{err}" if err.strip() else ""), flush=True)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)

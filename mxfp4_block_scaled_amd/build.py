"""Build the HIP library libmxfp4moe.so in-tree for gfx950 with hipcc.

Every source under csrc/ is compiled to an object in csrc/_build/ (in
parallel), then linked into mxfp4_block_scaled_amd/libmxfp4moe.so. Always
rebuilds (no stale-object logic): a build takes well under a minute.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "libmxfp4moe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
    "-Wall",
    "-Wno-unused-function",
]
SOURCES = ["quantize.hip", "route.hip", "gemm.hip", "gemm_stream.hip", "gemm_tile.hip", "gemm_wide.hip", "gemm_f8ring.hip", "gemm_w4a16.hip", "gemm_q8.hip", "fc2_combine.hip", "combine.hip", "ceilings.hip", "abi.cpp", "noalloc.hip"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    msgs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if msgs and verbose:
        print(msgs, flush=True)
    return obj


def build(verbose=False):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
